"""ctypes binding of ``libtokenweave.so`` (argument marshalling only).

Every step of the fused path runs in the library's HIP kernels; this module
only turns torch tensors into device pointers and the current torch stream
into a ``hipStream_t``, and turns status codes into exceptions.  torch is
imported before the library is loaded so that both share the one HIP runtime
already in the process.

There is no CPU fallback: if the library is not built, or a tensor is not on
a GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence, Union

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtokenweave.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "tokenweave.h")

TW_OK, TW_ERR_INVALID_ARG, TW_ERR_UNSUPPORTED, TW_ERR_DEVICE = 0, 1, 2, 3
TW_F32, TW_BF16 = 0, 1
TW_MAX_PARTIALS = 16
TW_PLAN_SPLIT, TW_PLAN_BELOW_THRESHOLD, TW_PLAN_SINGLE_WAVE = 0, 1, 2
TW_PLAN_NO_FEASIBLE_OFFSET, TW_PLAN_EMPTY = 3, 4
TW_PLAN_MEASURED_SPLIT, TW_PLAN_MEASURED_UNSPLIT, TW_PLAN_MEASURED_OVER_WAVES = 5, 6, 7

PLAN_REASONS = {0: "split", 1: "below_threshold", 2: "single_wave", 3: "no_feasible_offset",
                4: "empty", 5: "measured_split", 6: "measured_unsplit",
                7: "measured_over_waves"}


class TokenWeaveError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"status {status}: {detail}")
        self.status = status
        self.detail = detail


class SplitProblem(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("tokens_per_cta", ctypes.c_int64),
                ("ctas_per_token_tile", ctypes.c_int64), ("num_cus", ctypes.c_int32),
                ("ctas_per_cu", ctypes.c_int32), ("min_split_tokens", ctypes.c_int64),
                ("offsets", ctypes.POINTER(ctypes.c_int32)), ("num_offsets", ctypes.c_int32)]


class LaunchInfo(ctypes.Structure):
    _fields_ = [("num_cus", ctypes.c_int32), ("threads_per_workgroup", ctypes.c_int32),
                ("vectors_per_thread", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("round_rows", ctypes.c_int64), ("rows_per_dispatch", ctypes.c_int64),
                ("dispatches", ctypes.c_int64)]


TW_KERNEL_ALL_AT_ONCE, TW_KERNEL_SEQUENCED, TW_KERNEL_STRIDED, TW_KERNEL_BOTH_SLOTS = 0, 1, 2, 3
KERNEL_NAMES = {-1: "none", 0: "all", 1: "seq", 2: "strided", 3: "both"}


class SplitEntry(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("offset", ctypes.c_int32)]


class SplitPlanResult(ctypes.Structure):
    _fields_ = [("prefix_tokens", ctypes.c_int64), ("suffix_tokens", ctypes.c_int64),
                ("offset", ctypes.c_int32), ("waves_unsplit", ctypes.c_int32),
                ("waves_prefix", ctypes.c_int32), ("waves_suffix", ctypes.c_int32),
                ("reason", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m reduce_rmsnorm_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    common = [ctypes.POINTER(vp), i32, vp, vp, vp, vp, i64, i64, ctypes.c_float, ctypes.c_int]
    lib.tw_fused_reduce_rmsnorm.argtypes = common + [vp]
    lib.tw_fused_reduce_rmsnorm.restype = ctypes.c_int
    lib.tw_fused_reduce_rmsnorm_grid.argtypes = common + [i32, vp]
    lib.tw_fused_reduce_rmsnorm_grid.restype = ctypes.c_int
    lib.tw_shard_rmsnorm.argtypes = common + [i32, vp]
    lib.tw_shard_rmsnorm.restype = ctypes.c_int
    lib.tw_reduce_partials.argtypes = [ctypes.POINTER(vp), i32, vp, i64, i64, ctypes.c_int, vp]
    lib.tw_reduce_partials.restype = ctypes.c_int
    lib.tw_add_rmsnorm.argtypes = [vp, vp, vp, vp, vp, i64, i64, ctypes.c_float, ctypes.c_int, vp]
    lib.tw_add_rmsnorm.restype = ctypes.c_int
    lib.tw_split_plan.argtypes = [ctypes.POINTER(SplitProblem), ctypes.POINTER(SplitPlanResult)]
    lib.tw_split_plan.restype = ctypes.c_int
    lib.tw_split_plan_measured.argtypes = [ctypes.POINTER(SplitProblem), ctypes.POINTER(SplitEntry),
                                           i32, ctypes.POINTER(SplitPlanResult)]
    lib.tw_split_plan_measured.restype = ctypes.c_int
    lib.tw_fused_launch_info.argtypes = [i32, i64, i64, ctypes.c_int, vp,
                                         ctypes.POINTER(LaunchInfo)]
    lib.tw_fused_launch_info.restype = ctypes.c_int
    lib.tw_status_string.argtypes = [ctypes.c_int]
    lib.tw_status_string.restype = ctypes.c_char_p
    lib.tw_last_error.argtypes = []
    lib.tw_last_error.restype = ctypes.c_char_p
    lib.tw_abi_version.argtypes = []
    lib.tw_abi_version.restype = ctypes.c_int32
    lib.tw_set_pointer_checks.argtypes = [i32]
    lib.tw_set_pointer_checks.restype = None
    _lib = lib
    return lib


def declared_functions(header: str = HEADER_PATH):
    """Names of the functions ``include/tokenweave.h`` declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tw_[a-z0-9_]+)\s*\(", text)))


def tw_set_pointer_checks(enabled: bool) -> None:
    """Turn the library's opt-in device-pointer verification on or off."""
    load_library().tw_set_pointer_checks(1 if enabled else 0)


def _check(status: int) -> None:
    if status != TW_OK:
        lib = load_library()
        raise TokenWeaveError(status, lib.tw_last_error().decode(errors="replace"))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TW_BF16
    if t.dtype == torch.float32:
        return TW_F32
    raise ValueError(f"unsupported dtype {t.dtype}; expected torch.bfloat16 or torch.float32")


def _as_list(partials: Union[torch.Tensor, Sequence[torch.Tensor]]):
    if isinstance(partials, torch.Tensor):
        if partials.dim() != 3:
            raise ValueError("a stacked partials tensor must be [N, T, h]")
        return [partials[i] for i in range(partials.shape[0])]
    return list(partials)


def _marshal(partials, residual, weight, out, residual_out):
    """Checks the tensors and returns (N, pointer array, T, h, out,
    residual_out).  Every tensor must be a contiguous [T, h] (weight: [h])
    tensor of the residual's dtype on the residual's GPU; ``partials`` is a
    list of [T, h] tensors or one [N, T, h] tensor whose [T, h] slices are
    contiguous (a stacked tensor is checked once, not per partial)."""
    if residual.dim() != 2:
        raise ValueError("residual must be [T, h]")
    shape, dt, dev = residual.shape, residual.dtype, residual.device
    T, h = shape
    if isinstance(partials, torch.Tensor):
        if partials.dim() != 3:
            raise ValueError("a stacked partials tensor must be [N, T, h]")
        n = partials.shape[0]
        if n < 1:
            raise ValueError("at least one partial is required")
        if partials.shape[1:] != shape:
            raise ValueError(f"partial shape {tuple(partials.shape[1:])} != residual shape {(T, h)}")
        if partials.device != dev or dev.type != "cuda":
            raise ValueError("every tensor must be on the residual's GPU (there is no CPU path)")
        if partials.dtype is not dt:
            raise ValueError("every tensor must share one dtype")
        if T * h > 0 and (partials.stride(2) != 1 or (T > 1 and partials.stride(1) != h)):
            raise ValueError("tensors must be contiguous (each [T, h] slice of the partials)")
        step = partials.stride(0) * partials.element_size()
        base = partials.data_ptr()
        ptrs = (ctypes.c_void_p * n)(*range(base, base + n * step, step)) if step else \
            (ctypes.c_void_p * n)(*([base] * n))
    else:
        parts = list(partials)
        n = len(parts)
        if not parts:
            raise ValueError("at least one partial is required")
        for q in parts:
            if q.shape != shape:
                raise ValueError(f"partial shape {tuple(q.shape)} != residual shape {(T, h)}")
            if q.device != dev or dev.type != "cuda":
                raise ValueError("every tensor must be on the residual's GPU (there is no CPU path)")
            if q.dtype is not dt:
                raise ValueError("every tensor must share one dtype")
            if not q.is_contiguous():
                raise ValueError("tensors must be contiguous")
        ptrs = (ctypes.c_void_p * n)(*[q.data_ptr() for q in parts])
    if dev.type != "cuda" or weight.device != dev:
        raise ValueError("every tensor must be on a GPU, the residual's (there is no CPU path)")
    if weight.dtype is not dt:
        raise ValueError("every tensor must share one dtype")
    if weight.shape != (h,):
        raise ValueError("weight must be [h]")
    if not residual.is_contiguous() or not weight.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if out is None:
        out = torch.empty_like(residual)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    for t in (out, residual_out):
        if t.shape != shape or t.dtype is not dt or t.device != dev or not t.is_contiguous():
            raise ValueError("out and residual_out must be contiguous [T, h] tensors like residual")
    return n, ptrs, T, h, out, residual_out


class _on_device:
    """Makes the tensors' GPU the current device for the call, and does
    nothing when it already is (the common case, which then costs no
    device switch)."""

    __slots__ = ("_ctx",)

    def __init__(self, device: torch.device):
        self._ctx = None
        if device.index is not None and device.index != torch.cuda.current_device():
            self._ctx = torch.cuda.device(device)

    def __enter__(self):
        if self._ctx is not None:
            self._ctx.__enter__()

    def __exit__(self, *exc):
        if self._ctx is not None:
            self._ctx.__exit__(*exc)


# torch's current stream of a device as its raw hipStream_t, without making a
# Stream object (a per-call cost); the public call where torch lacks it.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(device: torch.device, stream: Optional[torch.cuda.Stream]):
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(device.index)
        stream = torch.cuda.current_stream(device)
    if stream.device != device:
        raise ValueError(f"the stream belongs to {stream.device}, the tensors to {device}")
    return stream.cuda_stream


def tw_fused_reduce_rmsnorm(partials, residual: torch.Tensor, weight: torch.Tensor, eps: float,
                            out: Optional[torch.Tensor] = None,
                            residual_out: Optional[torch.Tensor] = None,
                            stream: Optional[torch.cuda.Stream] = None):
    """Fused reduce + residual-add + RMSNorm over every row; returns
    ``(out, residual_out)``.  ``partials`` is a list of [T, h] tensors or one
    stacked [N, T, h] tensor."""
    lib = load_library()
    n, ptrs, T, h, out, residual_out = _marshal(partials, residual, weight, out, residual_out)
    with _on_device(residual.device):
        _check(lib.tw_fused_reduce_rmsnorm(ptrs, n, residual.data_ptr(), weight.data_ptr(),
                                           out.data_ptr(), residual_out.data_ptr(), T, h,
                                           float(eps), _dtype_code(residual),
                                           _stream_handle(residual.device, stream)))
    return out, residual_out


def tw_fused_reduce_rmsnorm_grid(partials, residual: torch.Tensor, weight: torch.Tensor,
                                 eps: float, num_workgroups: int,
                                 out: Optional[torch.Tensor] = None,
                                 residual_out: Optional[torch.Tensor] = None,
                                 stream: Optional[torch.cuda.Stream] = None):
    """The fused step on at most ``num_workgroups`` workgroups, each taking
    ceil(T / G) consecutive rows; bit-identical to tw_fused_reduce_rmsnorm."""
    lib = load_library()
    n, ptrs, T, h, out, residual_out = _marshal(partials, residual, weight, out, residual_out)
    with _on_device(residual.device):
        _check(lib.tw_fused_reduce_rmsnorm_grid(ptrs, n, residual.data_ptr(),
                                                weight.data_ptr(), out.data_ptr(),
                                                residual_out.data_ptr(), T, h, float(eps),
                                                _dtype_code(residual), int(num_workgroups),
                                                _stream_handle(residual.device, stream)))
    return out, residual_out


def tw_shard_rmsnorm(partials, residual: torch.Tensor, weight: torch.Tensor, eps: float,
                     shard_index: int, out: Optional[torch.Tensor] = None,
                     residual_out: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None):
    """The fused step on rows [floor(k*T/N), floor((k+1)*T/N)) of full-size
    buffers (N = number of partials); other rows of out/residual_out are left
    as they were."""
    lib = load_library()
    n, ptrs, T, h, out, residual_out = _marshal(partials, residual, weight, out, residual_out)
    with _on_device(residual.device):
        _check(lib.tw_shard_rmsnorm(ptrs, n, residual.data_ptr(), weight.data_ptr(),
                                    out.data_ptr(), residual_out.data_ptr(), T, h, float(eps),
                                    _dtype_code(residual), int(shard_index),
                                    _stream_handle(residual.device, stream)))
    return out, residual_out


def tw_fused_launch_info(num_partials: int, num_tokens: int, hidden: int,
                         dtype: torch.dtype = torch.bfloat16,
                         stream: Optional[torch.cuda.Stream] = None) -> dict:
    """How tw_fused_reduce_rmsnorm would launch a call of this shape on
    ``stream`` (host only): the CUs counted for the stream, the geometry, the
    round of resident workgroups, the dispatches and the first dispatch's
    kernel ("all", "seq", "strided" or "both" in ``kernel_name``).  Without a GPU (or
    with ``stream=None``) the stream is the null stream."""
    lib = load_library()
    code = TW_BF16 if dtype == torch.bfloat16 else TW_F32 if dtype == torch.float32 else None
    if code is None:
        raise ValueError(f"unsupported dtype {dtype}")
    handle = ctypes.c_void_p(stream.cuda_stream) if stream is not None else None
    info = LaunchInfo()
    _check(lib.tw_fused_launch_info(num_partials, num_tokens, hidden, code, handle,
                                    ctypes.byref(info)))
    d = {f: getattr(info, f) for f, _ in LaunchInfo._fields_}
    d["kernel_name"] = KERNEL_NAMES[d["kernel"]]
    return d


def tw_reduce_partials(partials, reduced: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Unfused comparator, step 1: reduced = round(sum of the partials)."""
    lib = load_library()
    parts = _as_list(partials)
    if not parts:
        raise ValueError("at least one partial is required")
    ref = parts[0]
    if ref.dim() != 2:
        raise ValueError("partials must be [T, h]")
    for p in parts:
        if not p.is_cuda or p.dtype != ref.dtype or not p.is_contiguous() or p.shape != ref.shape \
                or p.device != ref.device:
            raise ValueError("partials must be contiguous tensors of one shape and dtype on one GPU")
    if reduced is None:
        reduced = torch.empty_like(ref)
    if reduced.shape != ref.shape or reduced.dtype != ref.dtype or not reduced.is_contiguous() \
            or reduced.device != ref.device:
        raise ValueError("reduced must be a contiguous tensor like the partials")
    T, h = ref.shape
    ptrs = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
    with _on_device(ref.device):
        _check(lib.tw_reduce_partials(ptrs, len(parts), reduced.data_ptr(), T, h,
                                      _dtype_code(ref), _stream_handle(ref.device, stream)))
    return reduced


def tw_add_rmsnorm(inp: torch.Tensor, residual: torch.Tensor, weight: torch.Tensor, eps: float,
                   out: Optional[torch.Tensor] = None, residual_out: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None):
    """Unfused comparator, step 2: standard two-pass residual-add + RMSNorm."""
    lib = load_library()
    _, _, T, h, out, residual_out = _marshal([inp], residual, weight, out, residual_out)
    with _on_device(residual.device):
        _check(lib.tw_add_rmsnorm(inp.data_ptr(), residual.data_ptr(), weight.data_ptr(),
                                  out.data_ptr(), residual_out.data_ptr(), T, h, float(eps),
                                  _dtype_code(residual), _stream_handle(residual.device, stream)))
    return out, residual_out


def tw_unfused_reduce_rmsnorm(partials, residual: torch.Tensor, weight: torch.Tensor, eps: float,
                              out: Optional[torch.Tensor] = None,
                              residual_out: Optional[torch.Tensor] = None,
                              reduced: Optional[torch.Tensor] = None,
                              stream: Optional[torch.cuda.Stream] = None):
    """The unfused sequence: tw_reduce_partials, then tw_add_rmsnorm.
    Returns (out, residual_out, reduced)."""
    if reduced is None:
        reduced = torch.empty_like(residual)
    tw_reduce_partials(partials, reduced=reduced, stream=stream)
    out, residual_out = tw_add_rmsnorm(reduced, residual, weight, eps, out=out,
                                       residual_out=residual_out, stream=stream)
    return out, residual_out, reduced


def _split_problem(num_tokens, tokens_per_cta, ctas_per_token_tile, num_cus, ctas_per_cu,
                   min_split_tokens, offsets):
    arr = None
    if offsets is not None:
        arr = (ctypes.c_int32 * len(offsets))(*offsets)
    prob = SplitProblem(num_tokens, tokens_per_cta, ctas_per_token_tile, num_cus, ctas_per_cu,
                        min_split_tokens,
                        ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)) if arr is not None else None,
                        len(offsets) if offsets is not None else 0)
    return prob, arr


def _plan_dict(res: SplitPlanResult) -> dict:
    return {f: getattr(res, f) for f, _ in SplitPlanResult._fields_}


def tw_split_plan(num_tokens: int, tokens_per_cta: int = 1, ctas_per_token_tile: int = 1,
                  num_cus: int = 256, ctas_per_cu: int = 1, min_split_tokens: int = 0,
                  offsets: Optional[Sequence[int]] = None) -> dict:
    """Wave-aware prefix/suffix split plan (host only)."""
    lib = load_library()
    prob, _keep = _split_problem(num_tokens, tokens_per_cta, ctas_per_token_tile, num_cus,
                                 ctas_per_cu, min_split_tokens, offsets)
    res = SplitPlanResult()
    _check(lib.tw_split_plan(ctypes.byref(prob), ctypes.byref(res)))
    return _plan_dict(res)


def split_table(measured) -> ctypes.Array:
    """A measured table ({token count: offset, -1 for whole}) as the C
    planner's ascending array of tw_split_entry."""
    items = sorted((int(t), int(off)) for t, off in dict(measured).items())
    return (SplitEntry * len(items))(*[SplitEntry(t, off) for t, off in items])


def tw_split_plan_measured(num_tokens: int, table, tokens_per_cta: int = 1,
                           ctas_per_token_tile: int = 1, num_cus: int = 256,
                           ctas_per_cu: int = 1, min_split_tokens: int = 0,
                           offsets: Optional[Sequence[int]] = None) -> dict:
    """The split plan with a measured per-shape table consulted first (host
    only).  ``table`` is a {token count: offset} mapping (-1: keep whole) or
    an array from :func:`split_table`."""
    lib = load_library()
    arr = table if isinstance(table, ctypes.Array) else split_table(table)
    prob, _keep = _split_problem(num_tokens, tokens_per_cta, ctas_per_token_tile, num_cus,
                                 ctas_per_cu, min_split_tokens, offsets)
    res = SplitPlanResult()
    _check(lib.tw_split_plan_measured(ctypes.byref(prob), arr, len(arr), ctypes.byref(res)))
    return _plan_dict(res)


def tw_fused_reduce_rmsnorm_split(partials, residual: torch.Tensor, weight: torch.Tensor,
                                  eps: float, prefix_tokens: int,
                                  out: Optional[torch.Tensor] = None,
                                  residual_out: Optional[torch.Tensor] = None,
                                  stream: Optional[torch.cuda.Stream] = None):
    """Split execution: two launches, rows [0, P) then [P, T), on one stream.
    The suffix launch gets every pointer advanced by P rows."""
    T = residual.shape[0]
    if not 0 <= prefix_tokens <= T:
        raise ValueError("prefix_tokens must lie in [0, T]")
    if out is None:
        out = torch.empty_like(residual)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    P = int(prefix_tokens)
    stacked = isinstance(partials, torch.Tensor) and partials.dim() == 3
    parts = partials if stacked else _as_list(partials)
    for lo, hi in ((0, P), (P, T)):
        piece = parts[:, lo:hi] if stacked else [p[lo:hi] for p in parts]
        tw_fused_reduce_rmsnorm(piece, residual[lo:hi], weight, eps,
                                out=out[lo:hi], residual_out=residual_out[lo:hi], stream=stream)
    return out, residual_out


class PreparedFused:
    """A fused launch with its arguments marshalled once.

    For loops that launch the same step on the same buffers (a serving loop, a
    benchmark): the tensors are checked and turned into pointers here, each
    call is then one C call on the given stream.  The C side still validates
    every call.  ``mode`` is "full", "shard" (needs ``shard_index``) or "grid"
    (needs ``num_workgroups``).  Keeps references to every tensor it uses.
    """

    def __init__(self, partials, residual, weight, eps: float, out: torch.Tensor,
                 residual_out: torch.Tensor, stream: Optional[torch.cuda.Stream] = None,
                 mode: str = "full", shard_index: int = 0, num_workgroups: int = 0):
        lib = load_library()
        n, ptrs, T, h, out, residual_out = _marshal(partials, residual, weight, out,
                                                    residual_out)
        self._keep = (partials, residual, weight, out, residual_out, ptrs, stream)
        self.out, self.residual_out = out, residual_out
        head = (ptrs, n, residual.data_ptr(), weight.data_ptr(), out.data_ptr(),
                residual_out.data_ptr(), T, h, ctypes.c_float(float(eps)), _dtype_code(residual))
        s = _stream_handle(residual.device, stream)
        if mode == "full":
            self._fn, self._args = lib.tw_fused_reduce_rmsnorm, head + (s,)
        elif mode == "shard":
            self._fn, self._args = lib.tw_shard_rmsnorm, head + (int(shard_index), s)
        elif mode == "grid":
            self._fn, self._args = lib.tw_fused_reduce_rmsnorm_grid, head + (int(num_workgroups), s)
        else:
            raise ValueError(f"unknown mode {mode!r}")

    def __call__(self) -> None:
        _check(self._fn(*self._args))


class SplitPlanCache:
    """Split plans by token count for one model/GEMM configuration: each
    count is planned once and then looked up, as the pages keep the chosen
    split of each shape in a table.

    ``measured`` optionally maps token counts to the offset an offline sweep
    found fastest (-1: keep the batch whole), the way the pages choose their
    offsets by timing.  The table is handed to tw_split_plan_measured, which
    applies a listed offset when its pieces meet the wave condition and plans
    every other count analytically; this class only stores the plans."""

    def __init__(self, measured: Optional[dict] = None, **problem):
        self._problem = problem
        self._table = split_table(measured or {})
        tw_split_plan_measured(0, self._table, **problem)    # validates table and problem
        self._plans = {}

    def __call__(self, num_tokens: int) -> dict:
        """The plan for ``num_tokens`` (a copy: changing it leaves the table
        alone)."""
        plan = self._plans.get(num_tokens)
        if plan is None:
            plan = tw_split_plan_measured(num_tokens, self._table, **self._problem)
            self._plans[num_tokens] = plan
        return dict(plan)


def split_table_from_sweep(rows) -> dict:
    """The offline table from a measured sweep: ``rows`` are records with
    "tokens" and "fastest" (the fastest offset, or -1 for unsplit), such as
    the "table" that ``bench.py --overlap`` reports.  Returns {tokens: offset}
    for SplitPlanCache(measured=...)."""
    return {int(r["tokens"]): int(r["fastest"]) for r in rows}
