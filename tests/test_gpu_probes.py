"""The measurement probes of libtw_bwprobe.so write exactly what they claim,
so the bytes the envelope counts are the bytes they move: the flat streams
(xor of the sources, plus the destination index k, into every destination;
a known pattern for the writes-only stream) and the schedule twins of the
fused kernel's row classes (the xor of a row's sources as residual_out, and
that xor plus the row's wave-ordered checksum as out), in both load orders.
Small buffers, checked element by element on the host."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from reduce_rmsnorm_amd.build import PROBE_LIB_PATH

pytestmark = pytest.mark.gpu

# Twin row classes: vectors per row -> (threads per workgroup, vectors per thread)
TWIN_CLASSES = {1024: (1024, 1), 512: (512, 1), 2048: (1024, 2)}


def _lib():
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    vpp = ctypes.POINTER(ctypes.c_void_p)
    lib.tw_probe_launch.argtypes = [ctypes.c_int, vpp, ctypes.c_int, vpp, ctypes.c_int,
                                    ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.tw_probe_launch.restype = ctypes.c_int
    lib.tw_probe_twin_launch.argtypes = [ctypes.c_int, ctypes.c_int, vpp, ctypes.c_int, vpp,
                                         ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.tw_probe_twin_launch.restype = ctypes.c_int
    return lib


def _tensors(n, nvec, seed):
    rng = np.random.default_rng(seed)
    host = [rng.integers(0, 2 ** 32, size=(nvec, 4), dtype=np.uint32) for _ in range(n)]
    dev = [torch.from_numpy(h.view(np.int32)).cuda() for h in host]
    return host, dev


def _ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _down(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return _lib()


@pytest.mark.parametrize("nsrc,nvec", [(3, 5000), (9, 4096), (17, 777)])
def test_flat_streams_write_what_they_read(lib, nsrc, nvec):
    print(f"[case] flat probes nsrc={nsrc} nvec={nvec}", flush=True)
    host, src = _tensors(nsrc, nvec, seed=nsrc)
    dst = [torch.zeros((nvec, 4), dtype=torch.int32, device="cuda") for _ in range(2)]
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.tw_probe_launch(0, _ptrs(src), nsrc, _ptrs(dst), 2, nvec, 64, stream) == 0
    torch.cuda.synchronize()
    x = np.bitwise_xor.reduce(np.stack(host), axis=0)
    for k in range(2):
        np.testing.assert_array_equal(_down(dst[k]), x + np.uint32(k))
    for t in dst:
        t.zero_()
    assert lib.tw_probe_launch(2, _ptrs(src), 0, _ptrs(dst), 2, nvec, 64, stream) == 0
    torch.cuda.synchronize()
    want = np.stack([np.arange(nvec, dtype=np.uint32), np.full(nvec, 1, np.uint32),
                     np.full(nvec, 2, np.uint32), np.full(nvec, 3, np.uint32)], axis=1)
    for k in range(2):
        np.testing.assert_array_equal(_down(dst[k]), want)


@pytest.mark.parametrize("row", sorted(TWIN_CLASSES))
@pytest.mark.parametrize("sequenced", [0, 1])
@pytest.mark.parametrize("nsrc", [2, 9, 17])
def test_schedule_twin_writes_both_outputs_of_every_row(lib, row, sequenced, nsrc):
    rows = 3
    nvec = rows * row
    print(f"[case] twin row={row} sequenced={sequenced} nsrc={nsrc}", flush=True)
    host, src = _tensors(nsrc, nvec, seed=100 + row + nsrc)
    out = torch.zeros((nvec, 4), dtype=torch.int32, device="cuda")
    rout = torch.zeros((nvec, 4), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.tw_probe_twin_launch(5, sequenced, _ptrs(src), nsrc, _ptrs([out, rout]), nvec, rows,
                                    stream) == 0
    torch.cuda.synchronize()
    x = np.bitwise_xor.reduce(np.stack(host), axis=0)          # [nvec, 4]
    np.testing.assert_array_equal(_down(rout), x)
    block, vpt = TWIN_CLASSES[row]
    want = np.empty_like(x)
    for r in range(rows):
        xr = x[r * row:(r + 1) * row]
        # lane 0 of wave w holds vector slots 64w + j*block; its checksum is the
        # xor of their first words, and the row's total adds the waves in order
        tot = np.uint64(0)
        for w in range(block // 64):
            c = np.uint32(0)
            for j in range(vpt):
                c ^= xr[64 * w + j * block, 0]
            tot += np.uint64(c)
        want[r * row:(r + 1) * row] = xr + np.uint32(int(tot) & 0xFFFFFFFF)
    np.testing.assert_array_equal(_down(out), want)
    # the reads-only twin writes nothing for data like this
    out.zero_()
    assert lib.tw_probe_twin_launch(6, sequenced, _ptrs(src), nsrc, _ptrs([out]), nvec, rows,
                                    stream) == 0
    torch.cuda.synchronize()
    assert not _down(out).any()


def test_twin_rejects_shapes_it_has_no_class_for(lib):
    host, src = _tensors(2, 3000, seed=1)
    out = torch.zeros((3000, 4), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    # 1000 vectors per row: no twin class
    assert lib.tw_probe_twin_launch(5, 1, _ptrs(src), 2, _ptrs([out, out]), 3000, 3, stream) == -1
    # nvec not a multiple of the grid
    assert lib.tw_probe_twin_launch(5, 1, _ptrs(src), 2, _ptrs([out, out]), 3000, 7, stream) == -1
