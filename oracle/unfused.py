"""fp64 oracle of the unfused comparator: a standalone reduction of the N
partials followed by a standard two-pass residual-add + RMSNorm (test
infrastructure only; see the package docstring for who may import it).

Sources: [Blog] "TokenWeave: Why Hiding Tensor-Parallel Communication Needs
Wave Arithmetic, Not Finer Tiles" -- section "What it buys" (the fused kernel
is measured against a standalone AllReduce plus a standalone RMSNorm) and
section "Fix two: RMSNorm was never insignificant" (after the AllReduce every
GPU holds the reduced tensor in memory; a standard RMSNorm reads it twice,
once for the variance and once to scale, and writes it once).

Steps, per row t, in the order the unfused flow runs them:

1. reduced = round(sum_i P_i[t, :])      -- the AllReduce writes its result in
                                            the storage dtype (rounded once)
2. x = reduced + R[t, :]                 -- residual add, stored as
   residual_out = round(x)                  the new residual (rounded once)
3. ms = sum_j x_j^2 / h, rs = 1/sqrt(ms + eps)   -- first read: the unrounded x
4. y = (round(x) * rs) * w               -- second read: the stored tensor

Reading: the first read's variance comes from the sum before it is stored
and the second read scales the stored (rounded) values, since the second pass
reads the tensor back from memory.  For float32 storage "round" is the float32
rounding of the float64 value.
"""

from __future__ import annotations

import numpy as np

from .rmsnorm import bf16_bits_to_f64, f32_to_f64, round_f64_to_bf16_bits


def _widen(a, dtype):
    return bf16_bits_to_f64(a) if dtype == "bf16" else f32_to_f64(a)


def _round(x64, dtype):
    """Round float64 to the storage dtype once; returns (stored, its float64 value)."""
    if dtype == "bf16":
        bits = round_f64_to_bf16_bits(x64)
        return bits, bf16_bits_to_f64(bits)
    v = np.asarray(x64, dtype=np.float64).astype(np.float32)
    return v, v.astype(np.float64)


def reduce_partials(partials, dtype):
    """Step 1 for every row: (stored reduced tensor, its float64 value)."""
    acc = np.zeros(np.asarray(partials[0]).shape, dtype=np.float64)
    for p in partials:
        acc = acc + _widen(p, dtype)
    return _round(acc, dtype)


def add_rmsnorm_two_pass(inp, residual, weight, eps, dtype):
    """Steps 2-4 for every row of a stored input tensor.

    Returns (y, x, x_stored64): float64 normalized output, float64 unrounded
    sum x, and the float64 value of the stored residual (round(x))."""
    inp = np.asarray(inp)
    T, h = inp.shape
    eps64 = float(np.float32(eps))
    w = _widen(weight, dtype)
    y = np.empty((T, h), dtype=np.float64)
    x = np.empty((T, h), dtype=np.float64)
    xs = np.empty((T, h), dtype=np.float64)
    for t in range(T):
        xt = _widen(inp[t], dtype) + _widen(residual[t], dtype)
        ms = np.sum(xt * xt) / h
        rs = 1.0 / np.sqrt(ms + eps64)
        _, stored = _round(xt, dtype)
        y[t] = (stored * rs) * w
        x[t] = xt
        xs[t] = stored
    return y, x, xs


def unfused_reduce_rmsnorm(partials, residual, weight, eps, dtype):
    """Both steps: returns (y, x, reduced_stored) with y and x as float64 and
    the stored reduced tensor (uint16 bf16 bits or float32)."""
    red, _ = reduce_partials(partials, dtype)
    y, x, _ = add_rmsnorm_two_pass(red, residual, weight, eps, dtype)
    return y, x, red
