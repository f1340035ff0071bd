"""Helpers of the GPU tests: moving seeded inputs to the device, reading
results back, and the tolerance checks.

Tolerances (derived from the arithmetic; the bf16 bound is the one the
workloads fix):

* float32 path: every element of out and residual_out within a relative
  error of 1e-5 of the float64 oracle; an exact zero must be a zero.
* bf16 path: (i) the bit pattern is at most one step (ordinal distance,
  +0 == -0) from the oracle rounded once to bf16, and (ii) the value is
  within 2^-8 relative of the float64 oracle.  (ii) is the relative form of
  one bf16 ulp and holds for normal numbers only; below the smallest normal
  bf16 (2^-126) a step is 2^-133 absolute, and (i) alone applies.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def upload(d: dict, device="cuda"):
    dt = d["dtype"]
    parts = to_device(d["partials"], dt, device)
    return parts, to_device(d["residual"], dt, device), to_device(d["weight"], dt, device)


def _ordinal(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def check(got: np.ndarray, ref64: np.ndarray, dtype: str, what: str) -> int:
    """Assert the tolerance; returns the number of elements that are not
    bit-identical to the oracle rounded to the storage type."""
    assert got.shape == ref64.shape, (what, got.shape, ref64.shape)
    if dtype == "bf16":
        want = oracle.round_f64_to_bf16_bits(ref64)
        dist = np.abs(_ordinal(got) - _ordinal(want))
        val = oracle.bf16_bits_to_f64(got)
        rel_bad = (np.abs(val - ref64) > 2.0 ** -8 * np.abs(ref64)) & (np.abs(ref64) >= 2.0 ** -126)
        bad = np.nonzero((dist > 1) | rel_bad)
        assert bad[0].size == 0, (
            f"{what}: {bad[0].size} elements outside 1 bf16 step / 2^-8; first at "
            f"{tuple(int(i[0]) for i in bad)} got {val[bad][0]!r} want {ref64[bad][0]!r}")
        return int(np.count_nonzero(dist))
    got64 = got.astype(np.float64)
    err = np.abs(got64 - ref64)
    bad = np.nonzero(err > 1e-5 * np.abs(ref64))
    assert bad[0].size == 0, (
        f"{what}: {bad[0].size} elements beyond 1e-5 relative; first at "
        f"{tuple(int(i[0]) for i in bad)} got {got64[bad][0]!r} want {ref64[bad][0]!r}")
    return int(np.count_nonzero(got64 != ref64.astype(np.float32)))
