"""The Python binding's own checks that need no GPU: tensors off the GPU are
refused before anything reaches the library (there is no CPU path)."""

import pytest
import torch

import reduce_rmsnorm_amd as tw


def _cpu_inputs(T=4, h=16, N=2):
    parts = torch.zeros(N, T, h, dtype=torch.bfloat16)
    res = torch.zeros(T, h, dtype=torch.bfloat16)
    w = torch.ones(h, dtype=torch.bfloat16)
    return parts, res, w


@pytest.mark.parametrize("call", [
    lambda p, r, w: tw.tw_fused_reduce_rmsnorm(p, r, w, 1e-5),
    lambda p, r, w: tw.tw_fused_reduce_rmsnorm_grid(p, r, w, 1e-5, 4),
    lambda p, r, w: tw.tw_shard_rmsnorm(p, r, w, 1e-5, shard_index=0),
    lambda p, r, w: tw.tw_fused_reduce_rmsnorm_split(p, r, w, 1e-5, 2),
    lambda p, r, w: tw.tw_unfused_reduce_rmsnorm(p, r, w, 1e-5),
    lambda p, r, w: tw.PreparedFused(p, r, w, 1e-5, torch.empty_like(r), torch.empty_like(r)),
])
def test_cpu_tensors_are_refused(call):
    p, r, w = _cpu_inputs()
    with pytest.raises(ValueError, match="GPU"):
        call(p, r, w)


def test_shape_errors_before_device_checks():
    p, r, w = _cpu_inputs()
    with pytest.raises(ValueError, match="at least one partial"):
        tw.tw_fused_reduce_rmsnorm([], r, w, 1e-5)
    with pytest.raises(ValueError, match=r"\[T, h\]"):
        tw.tw_fused_reduce_rmsnorm(p, r.reshape(1, 4, 16), w, 1e-5)
