"""One tensor-parallel layer step on one GPU: the row-parallel GEMM that
produces this rank's partial, then the fused reduce + residual-add + RMSNorm
over the N partials -- run either one after the other, or split in two and
overlapped on two streams as TokenWeave does.

Sources: [Blog] "TokenWeave: Why Hiding Tensor-Parallel Communication Needs
Wave Arithmetic, Not Finer Tiles", section "Fix one: split at wave
boundaries, unequally" (split the batch in two, prefix = half + offset,
suffix = half - offset; offsets swept offline per shape), and [Guide]
"TokenWeave Guide: Compute-Communication Overlap for LLMs", section "The
Mathematics of Token-Splitting and Overlap" (while the compute stream runs
the second chunk's GEMM, the other stream runs the first chunk's fused
kernel).

Timeline of the split step (stream A computes, stream B normalizes):

    A:  GEMM(prefix) --e1--> GEMM(suffix) --e2-->
    B:             wait e1 -> fused(prefix) -> wait e2 -> fused(suffix)

The GEMM is a plain library GEMM (``torch.mm``: hipBLASLt/rocBLAS), which
writes the rank's partial P_0 in place; partials 1..N-1 stand for the peers'
and are already resident.  The fused kernels are this library's.  Both
streams keep the default priority.

The pages give the fused kernel a few SMs and leave the GEMM the rest ([Blog],
"Fix two": the kernel saturates the link on a small fraction of the SMs).
``MaskedStream`` is the MI355X tool for that partition: a HIP stream whose
kernels may only run on a chosen set of CUs (``hipExtStreamCreateWithCUMask``).
"""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from ._lib import tw_fused_reduce_rmsnorm, tw_fused_reduce_rmsnorm_grid

NUM_MASK_BITS = 256


def _hip_runtime() -> ctypes.CDLL:
    # torch has already loaded the HIP runtime under this soname; dlopen returns
    # that same instance, so streams made here are usable by torch and by this
    # library's launches.
    torch.cuda.init()
    hip = None
    for name in ("libamdhip64.so.7", "libamdhip64.so"):
        try:
            hip = ctypes.CDLL(name)
            break
        except OSError:
            continue
    if hip is None:
        raise RuntimeError("the HIP runtime library (libamdhip64.so) is not loadable")
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    hip.hipExtStreamCreateWithCUMask.restype = ctypes.c_int
    hip.hipExtStreamGetCUMask.argtypes = [ctypes.c_void_p, ctypes.c_uint32,
                                          ctypes.POINTER(ctypes.c_uint32)]
    hip.hipExtStreamGetCUMask.restype = ctypes.c_int
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    hip.hipStreamDestroy.restype = ctypes.c_int
    return hip


def mask_words(bits: Sequence[int], num_bits: int = NUM_MASK_BITS) -> list:
    """CU-mask bit indices -> the 32-bit words ``hipExtStreamCreateWithCUMask``
    takes (bit b is bit b % 32 of word b // 32)."""
    words = [0] * ((num_bits + 31) // 32)
    for b in bits:
        if not 0 <= b < num_bits:
            raise ValueError(f"CU mask bit {b} outside [0, {num_bits})")
        words[b // 32] |= 1 << (b % 32)
    return words


class MaskedStream:
    """A HIP stream (default priority) restricted to the CUs whose mask bits
    are given, wrapped as a torch stream (``.stream``).  ``close()`` waits for
    the stream's work and destroys it."""

    def __init__(self, bits: Sequence[int], num_bits: int = NUM_MASK_BITS):
        bits = sorted(set(bits))
        if not bits:
            raise ValueError("a CU mask needs at least one CU")
        self.bits = bits
        self._hip = _hip_runtime()
        words = mask_words(bits, num_bits)
        arr = (ctypes.c_uint32 * len(words))(*words)
        handle = ctypes.c_void_p()
        rc = self._hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), len(words), arr)
        if rc != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask failed with HIP error {rc}")
        self._handle = handle.value
        self.stream = torch.cuda.ExternalStream(self._handle)

    def mask(self) -> list:
        """The mask as the runtime holds it (32-bit words)."""
        n = (NUM_MASK_BITS + 31) // 32
        arr = (ctypes.c_uint32 * n)()
        rc = self._hip.hipExtStreamGetCUMask(self._handle, n, arr)
        if rc != 0:
            raise RuntimeError(f"hipExtStreamGetCUMask failed with HIP error {rc}")
        return list(arr)

    def close(self):
        if self._handle is not None:
            self.stream.synchronize()
            self._hip.hipStreamDestroy(self._handle)
            self._handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


class LayerStep:
    """Buffers for one layer step: activations X [T, K], weight W [K, h],
    ``sets`` rotating sets of partials [N, T, h] (partial 0 is the GEMM
    output), residual, outputs; RMSNorm weight [h]."""

    def __init__(self, num_tokens: int, hidden: int, k_dim: int, num_partials: int,
                 eps: float = 1e-5, sets: int = 2, device="cuda", seed: int = 0,
                 dtype=torch.bfloat16):
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        T, h, K, N = num_tokens, hidden, k_dim, num_partials
        self.T, self.h, self.K, self.N, self.eps = T, h, K, N, eps
        self.x = (torch.randn(T, K, device=device, generator=g) * 0.5).to(dtype)
        self.w_gemm = (torch.randn(K, h, device=device, generator=g) / K ** 0.5).to(dtype)
        self.weight = (1 + 0.05 * torch.randn(h, device=device, generator=g)).to(dtype)
        self.sets = []
        for _ in range(sets):
            parts = (torch.randn(N, T, h, device=device, generator=g) * 0.5).to(dtype)
            res = torch.randn(T, h, device=device, generator=g).to(dtype)
            self.sets.append((parts, res, torch.empty_like(res), torch.empty_like(res)))

    def _gemm(self, i: int, lo: int, hi: int):
        parts = self.sets[i % len(self.sets)][0]
        if hi > lo:
            torch.mm(self.x[lo:hi], self.w_gemm, out=parts[0, lo:hi])

    def _fused(self, i: int, lo: int, hi: int, stream, workgroups: Optional[int]):
        parts, res, out, rout = self.sets[i % len(self.sets)]
        if hi <= lo:
            return
        p = [parts[k, lo:hi] for k in range(self.N)]
        if workgroups is None:
            tw_fused_reduce_rmsnorm(p, res[lo:hi], self.weight, self.eps, out=out[lo:hi],
                                    residual_out=rout[lo:hi], stream=stream)
        else:
            tw_fused_reduce_rmsnorm_grid(p, res[lo:hi], self.weight, self.eps, workgroups,
                                         out=out[lo:hi], residual_out=rout[lo:hi], stream=stream)

    def run_unsplit(self, i: int, stream_a, workgroups: Optional[int] = None):
        """GEMM over every row, then the fused step, both on stream A."""
        with torch.cuda.stream(stream_a):
            self._gemm(i, 0, self.T)
            self._fused(i, 0, self.T, stream_a, workgroups)

    def run_split(self, i: int, prefix: int, stream_a, stream_b,
                  workgroups: Optional[int] = None):
        """The overlapped two-piece step; returns with stream B holding the
        last work (callers join it back to A)."""
        T = self.T
        e1 = torch.cuda.Event()
        e2 = torch.cuda.Event()
        with torch.cuda.stream(stream_a):
            self._gemm(i, 0, prefix)
            e1.record(stream_a)
            self._gemm(i, prefix, T)
            e2.record(stream_a)
        stream_b.wait_event(e1)
        self._fused(i, 0, prefix, stream_b, workgroups)
        stream_b.wait_event(e2)
        self._fused(i, prefix, T, stream_b, workgroups)

    def outputs(self, i: int):
        return self.sets[i % len(self.sets)]


def capture(step, stream_a, stream_b, i: int) -> torch.cuda.CUDAGraph:
    """Record ``step(i)`` (GEMMs, events and fused launches on both streams)
    into one HIP graph.  Stream B forks from stream A and joins back inside
    the capture.  The step records no memset of its own.  Run the step
    eagerly once beforehand: the GEMM library sets itself up per shape on
    first use, which is not allowed during capture."""
    g = torch.cuda.CUDAGraph()
    stream_a.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=stream_a):
        stream_b.wait_stream(stream_a)
        step(i)
        stream_a.wait_stream(stream_b)
    torch.cuda.synchronize()
    return g


def time_graphs(graphs, stream_a, iters: int, warmup: int = 3) -> float:
    """Mean microseconds per replay, cycling through ``graphs``."""
    with torch.cuda.stream(stream_a):
        for i in range(warmup):
            graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream_a):
        start.record(stream_a)
        for i in range(iters):
            graphs[i % len(graphs)].replay()
        end.record(stream_a)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / iters


def time_steps(step, stream_a, stream_b, iters: int, warmup: int = 5) -> float:
    """Mean microseconds per step for ``step(i)`` (which may use both
    streams), timed on stream A after joining stream B back into it."""
    for i in range(warmup):
        step(i)
        stream_a.wait_stream(stream_b)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream_a)
    for i in range(iters):
        stream_b.wait_stream(stream_a)
        step(i)
        stream_a.wait_stream(stream_b)
    end.record(stream_a)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / iters
