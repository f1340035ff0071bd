"""Seeded synthetic inputs for the fused reduce + residual-add + RMSNorm step.

This module is the only code that both the oracle side (tests) and the HIP
side (tests, bench) use.  It holds none of the method's arithmetic: it draws
normal variates, rounds them once to the storage dtype, and builds structured
special inputs (constant, one-hot, zero and integer-scaled rows).

Workloads (shapes from the models the TokenWeave pages serve -- Llama-3-70B,
Qwen2.5-72B, Mixtral, Llama-3.1-405B hidden sizes, 1K-8K tokens; the pages'
own end-to-end traces and weights are not used, these draws stand in for them):

==========  =====  =====  =====  ==  =============================
name        dtype  T      h      N   notes
==========  =====  =====  =====  ==  =============================
tiny        f32    64     512    2   partials, residual ~N(0,1)
llama70b    bf16   1024   8192   8   the headline shape
qwen72b     bf16   4096   8192   8   eps 1e-6, run split in two
mixtral     bf16   8192   4096   8   1% of rows' partials x100
llama405b   bf16   2048   16384  8   shard mode, every k
==========  =====  =====  =====  ==  =============================

bf16 partials ~N(0, 0.5), residual ~N(0, 1), weight ~N(1, 0.05); the fp32
tiny case uses partials and residual ~N(0, 1) and weight ~N(1, 0.1).

Recipe: ``numpy.random.default_rng(seed)`` with seed = the config's index
(0..4); draw order partials 0..N-1, residual, weight, then (mixtral only) the
outlier rows ``rng.choice(T, round(0.01*T), replace=False)``.  Draws are
float32 (``standard_normal(dtype=float32) * sigma + mu``); outlier rows of
every partial are multiplied by 100 in float32; then each tensor is rounded
once, round-to-nearest-even, to bf16 bits (uint16).  Both sides see the same
bytes, so no cross-platform generator agreement is needed.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    dtype: str              # "bf16" or "f32"
    num_tokens: int         # T
    hidden: int             # h
    num_partials: int       # N
    eps: float
    partial_sigma: float
    residual_sigma: float = 1.0
    weight_mean: float = 1.0
    weight_sigma: float = 0.05
    outlier_fraction: float = 0.0
    outlier_scale: float = 100.0
    modes: tuple = field(default=("full",))

    @property
    def itemsize(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def algorithmic_bytes(self, rows: Optional[int] = None) -> int:
        """(N + 1) reads + 2 writes of [rows, h] elements."""
        t = self.num_tokens if rows is None else rows
        return (self.num_partials + 3) * t * self.hidden * self.itemsize


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        Workload("tiny", 0, "f32", 64, 512, 2, 1e-5, 1.0, 1.0, 1.0, 0.1,
                 modes=("full", "shard")),
        Workload("llama70b", 1, "bf16", 1024, 8192, 8, 1e-5, 0.5,
                 modes=("full", "shard")),
        Workload("qwen72b", 2, "bf16", 4096, 8192, 8, 1e-6, 0.5,
                 modes=("full", "split")),
        Workload("mixtral", 3, "bf16", 8192, 4096, 8, 1e-5, 0.5,
                 outlier_fraction=0.01, modes=("full", "shard")),
        Workload("llama405b", 4, "bf16", 2048, 16384, 8, 1e-5, 0.5,
                 modes=("full", "shard")),
    )
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 bit patterns, nearest-even.

    Adds 0x7FFF plus the lowest kept bit to the float32 bits and drops the low
    16 bits: halfway cases go to the even neighbour.  Only used on finite
    draws (no NaN handling needed).
    """
    b = np.asarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    return np.ascontiguousarray(a32, dtype=np.float32)


def make_inputs(workload, num_tokens: Optional[int] = None, hidden: Optional[int] = None,
                seed: Optional[int] = None) -> dict:
    """Draw one batch for ``workload`` (a :class:`Workload` or its name).

    ``num_tokens``/``hidden`` shrink the shape for quick cases while keeping
    the workload's distributions.  Returns a dict with ``partials`` [N, T, h],
    ``residual`` [T, h], ``weight`` [h] (uint16 bf16 bits or float32),
    ``eps``, ``dtype``, ``outlier_rows`` and the workload.
    """
    wl = WORKLOADS[workload] if isinstance(workload, str) else workload
    T = wl.num_tokens if num_tokens is None else int(num_tokens)
    h = wl.hidden if hidden is None else int(hidden)
    N = wl.num_partials
    rng = np.random.default_rng(wl.index if seed is None else seed)
    f32 = np.float32
    parts = np.empty((N, T, h), dtype=np.float32)
    for i in range(N):
        parts[i] = rng.standard_normal((T, h), dtype=np.float32) * f32(wl.partial_sigma)
    res = rng.standard_normal((T, h), dtype=np.float32) * f32(wl.residual_sigma)
    w = rng.standard_normal(h, dtype=np.float32) * f32(wl.weight_sigma) + f32(wl.weight_mean)
    outliers = np.zeros(0, dtype=np.int64)
    if wl.outlier_fraction > 0 and T > 0:
        k = int(round(wl.outlier_fraction * T))
        outliers = np.sort(rng.choice(T, k, replace=False)).astype(np.int64)
        parts[:, outliers, :] *= f32(wl.outlier_scale)
    return dict(partials=_store(parts, wl.dtype), residual=_store(res, wl.dtype),
                weight=_store(w, wl.dtype), eps=wl.eps, dtype=wl.dtype,
                outlier_rows=outliers, workload=wl)


def _from_f32(dtype, *arrays):
    return tuple(_store(np.asarray(a, dtype=np.float32), dtype) for a in arrays)


def integer_scaled_inputs(num_partials: int, num_tokens: int, hidden: int, dtype: str,
                          kmax: int = 64, seed: int = 0) -> dict:
    """Inputs whose values are k/16 with integer k in [-kmax, kmax].

    Every such value is exact in bf16 and float32 (|k| <= 64 needs 7 bits), and
    so is every partial sum of up to 17 of them: the reduction is exact in any
    order.  Weight is drawn the same way but kept away from zero.
    """
    rng = np.random.default_rng(seed)
    parts = rng.integers(-kmax, kmax + 1, (num_partials, num_tokens, hidden)) / 16.0
    res = rng.integers(-kmax, kmax + 1, (num_tokens, hidden)) / 16.0
    w = rng.integers(8, 33, hidden) / 16.0
    p, r, ww = _from_f32(dtype, parts, res, w)
    return dict(partials=p, residual=r, weight=ww, dtype=dtype)


def special_rows_inputs(num_partials: int, num_tokens: int, hidden: int, dtype: str,
                        constants=(2.0 ** -10, -2.0 ** -8, 2.0 ** -6, -1.0, 2.0 ** 8),
                        seed: int = 0) -> dict:
    """Structured rows: each row is a zero row, a constant row or a one-hot row.

    Row t uses pattern t % (2 * len(constants) + 1): 0 is a zero row, the next
    len(constants) are constant rows x_j = c (carried entirely by partial 0),
    the rest are one-hot rows x = c * e_j with j = (7 * t) % h, carried by the
    residual.  All other tensors are exact zeros.  Weight is 1 for constant
    rows to apply the closed form directly, and drawn from {0.5 .. 2} in
    steps of 1/16 otherwise; two weights are returned (``weight_one`` and
    ``weight``).  ``kind`` and ``value`` describe each row.
    """
    rng = np.random.default_rng(seed)
    nc = len(constants)
    parts = np.zeros((num_partials, num_tokens, hidden), dtype=np.float32)
    res = np.zeros((num_tokens, hidden), dtype=np.float32)
    kind = np.zeros(num_tokens, dtype=np.int64)     # 0 zero, 1 constant, 2 one-hot
    value = np.zeros(num_tokens, dtype=np.float64)
    hot = np.zeros(num_tokens, dtype=np.int64)
    for t in range(num_tokens):
        p = t % (2 * nc + 1)
        if p == 0:
            continue
        c = constants[(p - 1) % nc]
        value[t] = c
        if p <= nc:
            kind[t] = 1
            parts[0, t, :] = c
        else:
            kind[t] = 2
            hot[t] = (7 * t) % hidden
            res[t, hot[t]] = c
    w = rng.integers(8, 33, hidden) / 16.0
    p, r, ww, w1 = _from_f32(dtype, parts, res, w, np.ones(hidden))
    return dict(partials=p, residual=r, weight=ww, weight_one=w1, dtype=dtype,
                kind=kind, value=value, hot=hot)
