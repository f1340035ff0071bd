"""fp64 oracle of the fused reduce + residual-add + RMSNorm step (test
infrastructure only; see the package docstring for who may import it).

What is computed, per token row t (the reading of the pages used here):

1. x = sum_i P_i[t, :] + R[t, :]
   -- [Blog] "TokenWeave: Why Hiding Tensor-Parallel Communication Needs Wave
   Arithmetic, Not Finer Tiles", section "Fix two: RMSNorm was never
   insignificant": the kernel sketch reduces the N tensor-parallel partials of
   this GPU's rows into a register-resident vector and then adds the residual
   in the same pass.
2. ms = (1/h) * sum_j x_j^2
   -- same sketch ("variance" divided by the hidden size, no mean subtracted)
   and [Guide] "TokenWeave Guide: Compute-Communication Overlap for LLMs",
   section "Fused AllReduce-RMSNorm: Bypassing Global Memory", the RMSNorm
   equation (the 1/D mean of squares under the root).
3. rs = 1 / sqrt(ms + eps)  (eps inside the root, same two sources).
4. y = (x * rs) * w  (scaled by the learnable weight gamma, elementwise).

Outputs are the normalized rows y and the updated residual x.  Everything is
computed in float64.  bf16 inputs are widened exactly (bits << 16 is the
float32 value, which float64 holds exactly).  The eps used is the float32 value
that crosses the library's C ABI, widened exactly.  For bf16 outputs the
reference is the float64 value rounded ONCE, directly, to bf16 with IEEE
round-to-nearest-even (:func:`round_f64_to_bf16_bits`); rounding through
float32 first would round twice.

Shard mode (same sketch section: after a token-boundary ReduceScatter each
GPU owns the final values of 1/N of the tokens and normalizes only those)
covers rows [floor(k*T/N), floor((k+1)*T/N)).  The per-row arithmetic is the
same as in full mode.
"""

from __future__ import annotations

from typing import Iterable, Sequence

import numpy as np

BF16 = "bf16"
F32 = "f32"


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64.

    A bf16 value is the upper half of a float32, so shifting the 16 bits left
    by 16 gives that float32 exactly; float64 represents every float32.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # NaN patterns widen to NaN
        return b.view(np.float32).astype(np.float64)


def f32_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of float32 values to float64."""
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def round_f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values directly to bf16 (IEEE round-to-nearest-even).

    bf16 has 8 significant bits (7 stored), exponent range of float32, and
    subnormals spaced 2**-133 apart.  For |x| = m * 2**e with 0.5 <= m < 1
    (``np.frexp``) the bf16 spacing in that binade is 2**(e-8); below the
    smallest normal (2**-126) it stays 2**-133.  Dividing by the spacing is
    exact (power of two), ``np.rint`` rounds half to even, and the rounded
    multiple of the spacing is exactly a bf16 value (hence a float32 value, whose
    upper 16 bits are the answer).  A result of 2**128 or more is infinity.
    NaN maps to the canonical quiet NaN with the input's sign.
    """
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.zeros(flat.shape, dtype=np.uint16)
    sign = np.signbit(flat)
    a = np.abs(flat)
    nan = np.isnan(a)
    inf = np.isinf(a)
    fin = ~(nan | inf)
    af = np.where(fin, a, 0.0)
    _, e = np.frexp(af)
    spacing_exp = np.maximum(e, -125) - 8
    k = np.rint(np.ldexp(af, -spacing_exp))           # exact scaling, RNE
    r = np.ldexp(k, spacing_exp)                       # exactly a bf16 value
    overflow = fin & (r >= 2.0 ** 128)
    ok = fin & ~overflow
    r32 = np.where(ok, r, 0.0).astype(np.float32)      # exact for every ok entry
    mag = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[ok] = mag[ok]
    out[inf | overflow] = 0x7F80
    out[nan] = 0x7FC0
    out |= np.where(sign, np.uint16(0x8000), np.uint16(0)).astype(np.uint16)
    return out.reshape(x.shape)


def _widen(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return bf16_bits_to_f64(a)
    if dtype == F32:
        return f32_to_f64(a)
    raise ValueError(f"unknown dtype {dtype!r}")


def shard_rows(num_tokens: int, num_shards: int, k: int) -> range:
    """Rows owned by shard k of N: [floor(k*T/N), floor((k+1)*T/N)).

    Multiplying before dividing gives every row to exactly one shard when N
    does not divide T (a reading: the pages only say each GPU owns its 1/N
    token shard, [Blog] section "Fix two").
    """
    if not (0 <= k < num_shards):
        raise ValueError("shard index out of range")
    return range((k * num_tokens) // num_shards, ((k + 1) * num_tokens) // num_shards)


def fused_reduce_rmsnorm(
    partials: Sequence[np.ndarray],
    residual: np.ndarray,
    weight: np.ndarray,
    eps: float,
    dtype: str,
    rows: Iterable[int] | None = None,
):
    """fp64 reference of the fused step for the given rows (default: all).

    ``partials`` is a sequence of N arrays [T, h] (uint16 bf16 bits or
    float32), ``residual`` is [T, h], ``weight`` is [h].  Returns
    ``(y, x, row_index)``: float64 arrays [len(rows), h] of the normalized
    output and of the updated residual, and the row indices they belong to.
    """
    residual = np.asarray(residual)
    T, h = residual.shape
    if rows is None:
        rows = range(T)
    rows = np.asarray(list(rows), dtype=np.int64)
    eps64 = float(np.float32(eps))        # the float32 eps that crosses the ABI
    w = _widen(weight, dtype)
    y = np.empty((rows.size, h), dtype=np.float64)
    x = np.empty((rows.size, h), dtype=np.float64)
    for n, t in enumerate(rows):
        xt = np.zeros(h, dtype=np.float64)
        for p in partials:                # step 1: reduce the N partials ...
            xt = xt + _widen(p[t], dtype)
        xt = xt + _widen(residual[t], dtype)   # ... then add the residual
        ms = np.sum(xt * xt) / h               # step 2: mean of squares
        rs = 1.0 / np.sqrt(ms + eps64)         # step 3: eps inside the root
        y[n] = (xt * rs) * w                   # step 4: scale, then weight
        x[n] = xt
    return y, x, rows


def shard_rmsnorm(partials, residual, weight, eps, dtype, shard_index, num_shards=None):
    """Shard mode: the fused step on the rows of shard k only.

    The shard count is the partial count N unless given.
    """
    n = len(partials) if num_shards is None else num_shards
    T = np.asarray(residual).shape[0]
    return fused_reduce_rmsnorm(partials, residual, weight, eps, dtype,
                                rows=shard_rows(T, n, shard_index))
