"""Oracle of the wave-aware prefix/suffix split planner (test infrastructure
only; see the package docstring for who may import it).

Source: [Blog] "TokenWeave: Why Hiding Tensor-Parallel Communication Needs
Wave Arithmetic, Not Finer Tiles".

* Section "The overlap trap": a GEMM launches some number of CTAs, each
  taking about one SM, and the GPU runs them in waves of as many CTAs as it has
  SMs; 300 CTAs on 132 SMs take three waves, two halves of 150 take two each.
* Section "Fix one: split at wave boundaries, unequally": the batch is split
  exactly twice; the condition is that the waves of the two pieces together do
  not exceed the waves of the unsplit batch; the prefix gets half + offset
  tokens and the suffix half - offset, with the offset drawn from
  {0, 64, 128, 192, 256, 512} and kept below half; a batch that is already a
  single wave is not split (all tokens go to the prefix); below a per-model
  token threshold (1K dense, 4K MoE) splitting is skipped.

Readings where the page is silent or its example disagrees with its rule:

* The page picks the offset by timing cuBLAS offline.  With no GEMM to time,
  the plan takes the smallest offset in the set whose two pieces meet the wave
  condition.  Because ceil(a/s) + ceil(b/s) >= ceil((a+b)/s), a feasible pair
  always has exactly the unsplit wave count, so "smallest feasible offset" is
  the only tie-break needed.
* The worked example's 132/168 split makes the prefix the smaller piece, while
  the rule gives prefix = half + offset >= half.  The example fixes wave counts
  only; the plan follows the rule (300 tokens-as-CTAs on 132 SMs gives 214/86).
* For odd T, half = floor(T/2) and suffix = T - prefix, so no token is lost.
* T equal to the threshold may split; only T below it skips.
* No feasible offset: no split (fuse only).
* The CTA count of the GEMM is modelled as ceil(M / tokens_per_cta) times the
  number of tiles across the output features, and a wave holds
  num_cus * ctas_per_cu CTAs (the page assumes one CTA per SM).
* A measured table (the page's per-shape lookup of the offset its offline
  timing found fastest) is consulted after the threshold and the one-wave
  rule, in the page's order.  Its offset is applied as half + offset, and it
  is still held to the wave condition: an entry whose two pieces would take
  more waves than the whole batch keeps the batch whole.  An entry of -1
  (the sweep found the whole batch fastest) keeps it whole too.
"""

from __future__ import annotations

import heapq
from typing import Sequence

DEFAULT_OFFSETS = (0, 64, 128, 192, 256, 512)

REASON_SPLIT = 0
REASON_BELOW_THRESHOLD = 1
REASON_SINGLE_WAVE = 2
REASON_NO_FEASIBLE_OFFSET = 3
REASON_EMPTY = 4
REASON_MEASURED_SPLIT = 5
REASON_MEASURED_UNSPLIT = 6
REASON_MEASURED_OVER_WAVES = 7


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def ctas(m: int, tokens_per_cta: int = 1, ctas_per_token_tile: int = 1) -> int:
    """CTAs a GEMM over m token rows launches under the tile model."""
    return _ceil_div(m, tokens_per_cta) * ctas_per_token_tile


def waves(m: int, tokens_per_cta: int = 1, ctas_per_token_tile: int = 1,
          num_cus: int = 256, ctas_per_cu: int = 1) -> int:
    """Waves of that GEMM: ceil(CTAs / CTAs resident per wave); 0 for m = 0."""
    return _ceil_div(ctas(m, tokens_per_cta, ctas_per_token_tile), num_cus * ctas_per_cu)


def simulate_waves(num_ctas: int, num_slots: int) -> int:
    """Brute-force scheduler: CTAs of equal duration are handed out one at a
    time to whichever slot frees first; count the distinct start times.

    This is an independent check of the ceil formula, not a use of it.
    """
    if num_ctas == 0:
        return 0
    free = [(0, i) for i in range(num_slots)]   # (time the slot is next free, slot)
    heapq.heapify(free)
    starts = set()
    for _ in range(num_ctas):
        t, slot = heapq.heappop(free)
        starts.add(t)
        heapq.heappush(free, (t + 1, slot))      # unit duration
    return len(starts)


def split_plan(num_tokens: int, tokens_per_cta: int = 1, ctas_per_token_tile: int = 1,
               num_cus: int = 256, ctas_per_cu: int = 1, min_split_tokens: int = 0,
               offsets: Sequence[int] | None = None) -> dict:
    """Plan the prefix/suffix token split, following the steps of [Blog]
    section "Fix one" in its order.

    Returns a dict with prefix_tokens, suffix_tokens, offset (-1 if not
    split), waves_unsplit, waves_prefix, waves_suffix and reason.
    """
    offs = DEFAULT_OFFSETS if offsets is None else tuple(offsets)
    T = num_tokens

    def wv(m):
        return waves(m, tokens_per_cta, ctas_per_token_tile, num_cus, ctas_per_cu)

    W = wv(T)

    def no_split(reason):
        return dict(prefix_tokens=T, suffix_tokens=0, offset=-1, waves_unsplit=W,
                    waves_prefix=W, waves_suffix=0, reason=reason)

    if T == 0:
        return no_split(REASON_EMPTY)
    if T < min_split_tokens:            # below the per-model threshold
        return no_split(REASON_BELOW_THRESHOLD)
    if W <= 1:                          # already one wave: everything to the prefix
        return no_split(REASON_SINGLE_WAVE)
    half = T // 2
    for off in offs:                    # offsets in the page's order
        if off >= half:                 # the page keeps off < half
            continue
        prefix = half + off
        suffix = T - prefix
        wp, ws = wv(prefix), wv(suffix)
        if wp + ws <= W:                # the wave condition
            return dict(prefix_tokens=prefix, suffix_tokens=suffix, offset=off,
                        waves_unsplit=W, waves_prefix=wp, waves_suffix=ws,
                        reason=REASON_SPLIT)
    return no_split(REASON_NO_FEASIBLE_OFFSET)


def split_plan_measured(num_tokens: int, table, tokens_per_cta: int = 1,
                        ctas_per_token_tile: int = 1, num_cus: int = 256, ctas_per_cu: int = 1,
                        min_split_tokens: int = 0, offsets: Sequence[int] | None = None) -> dict:
    """Plan the split with a measured per-shape table, as [Blog] section
    "Fix one" keeps the offset its offline timing sweep chose for each shape.

    ``table`` maps token counts to the measured offset (-1: the whole batch
    was fastest).  The threshold and the one-wave rule come first; a count
    with no entry gets the analytic plan of :func:`split_plan`.
    """
    T = num_tokens

    def wv(m):
        return waves(m, tokens_per_cta, ctas_per_token_tile, num_cus, ctas_per_cu)

    for t, off in dict(table).items():
        if t < 1 or not (off == -1 or 0 <= off < t // 2):
            raise ValueError(f"table entry {t}: offset {off} outside [0, T/2) or -1")
    W = wv(T)

    def no_split(reason):
        return dict(prefix_tokens=T, suffix_tokens=0, offset=-1, waves_unsplit=W,
                    waves_prefix=W, waves_suffix=0, reason=reason)

    if T == 0:
        return no_split(REASON_EMPTY)
    if T < min_split_tokens:
        return no_split(REASON_BELOW_THRESHOLD)
    if W <= 1:
        return no_split(REASON_SINGLE_WAVE)
    if T not in dict(table):
        return split_plan(T, tokens_per_cta, ctas_per_token_tile, num_cus, ctas_per_cu,
                          min_split_tokens, offsets)
    off = dict(table)[T]
    if off == -1:                       # the sweep kept this shape whole
        return no_split(REASON_MEASURED_UNSPLIT)
    prefix = T // 2 + off
    suffix = T - prefix
    wp, ws = wv(prefix), wv(suffix)
    if wp + ws > W:                     # the wave condition still holds the plan
        return no_split(REASON_MEASURED_OVER_WAVES)
    return dict(prefix_tokens=prefix, suffix_tokens=suffix, offset=off, waves_unsplit=W,
                waves_prefix=wp, waves_suffix=ws, reason=REASON_MEASURED_SPLIT)
