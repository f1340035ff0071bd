"""Parity of the HIP path (called through the C ABI) with the float64 oracle,
element by element, on seeded inputs; bit-identity invariants; edge cases.

Every kernel launch here is preceded by a flushed line naming the case."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import reduce_rmsnorm_amd as tw
from synthetic import WORKLOADS, integer_scaled_inputs, make_inputs, special_rows_inputs
from tests._gpu_util import check, to_device, to_host, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tw.load_library()
    torch.cuda.init()


def say(*a):
    print("[case]", *a, flush=True)


def _run_full(parts, res, w, eps):
    out, rout = tw.tw_fused_reduce_rmsnorm(parts, res, w, eps)
    torch.cuda.synchronize()
    return to_host(out), to_host(rout)


def _oracle(d, rows=None):
    return oracle.fused_reduce_rmsnorm(list(d["partials"]), d["residual"], d["weight"], d["eps"],
                                       d["dtype"], rows=rows)


# ------------------------------------------------------------- workloads ----

@pytest.mark.parametrize("name", list(WORKLOADS))
def test_full_mode_matches_oracle(name):
    d = make_inputs(name)
    wl = d["workload"]
    say(f"full {name}: T={wl.num_tokens} h={wl.hidden} N={wl.num_partials} {wl.dtype} seed={wl.index}")
    parts, res, w = upload(d)
    out, rout = _run_full(parts, res, w, d["eps"])
    y, x, _ = _oracle(d)
    n_y = check(out, y, d["dtype"], f"{name} out")
    n_x = check(rout, x, d["dtype"], f"{name} residual_out")
    say(f"{name}: out not bit-exact {n_y}/{y.size}, residual_out not bit-exact {n_x}/{x.size}")


@pytest.mark.parametrize("name", ["tiny", "llama70b", "mixtral", "llama405b"])
def test_shard_mode_matches_full_and_leaves_other_rows(name):
    d = make_inputs(name)
    wl = d["workload"]
    N, T = wl.num_partials, wl.num_tokens
    parts, res, w = upload(d)
    say(f"full {name} (reference for shards)")
    out_full, rout_full = _run_full(parts, res, w, d["eps"])
    y, x, _ = _oracle(d) if name != "llama405b" else (None, None, None)
    for k in range(N):
        rows = oracle.shard_rows(T, N, k)
        out = torch.full_like(res, float("nan"))
        rout = torch.full_like(res, float("nan"))
        say(f"shard {name} k={k} rows [{rows.start}, {rows.stop})")
        tw.tw_shard_rmsnorm(parts, res, w, d["eps"], k, out=out, residual_out=rout)
        torch.cuda.synchronize()
        o, r = to_host(out), to_host(rout)
        sl = slice(rows.start, rows.stop)
        np.testing.assert_array_equal(o[sl], out_full[sl])      # bit-identical to full mode
        np.testing.assert_array_equal(r[sl], rout_full[sl])
        if y is not None:
            check(o[sl], y[sl], d["dtype"], f"{name} shard {k} out")
            check(r[sl], x[sl], d["dtype"], f"{name} shard {k} residual_out")
        other = np.ones(T, bool)
        other[sl] = False
        canary = oracle.bf16_bits_to_f64(o[other]) if d["dtype"] == "bf16" else o[other]
        assert np.isnan(canary).all()
        canary = oracle.bf16_bits_to_f64(r[other]) if d["dtype"] == "bf16" else r[other]
        assert np.isnan(canary).all()


# The planner settings the benchmark uses for each workload: 256 x 256 GEMM
# tiles across h, one per CU on 256 CUs; the MoE threshold for mixtral.
SPLIT_PLANS = {"qwen72b": 1024, "mixtral": 4096, "llama405b": 1024}


@pytest.mark.parametrize("name", list(SPLIT_PLANS))
def test_split_launches_equal_one_launch_for_every_offset(name):
    d = make_inputs(name)
    T, h = d["workload"].num_tokens, d["workload"].hidden
    parts, res, w = upload(d)
    say(f"full {name} (reference for splits)")
    out_full, rout_full = _run_full(parts, res, w, d["eps"])
    kw = dict(tokens_per_cta=256, ctas_per_token_tile=h // 256, num_cus=256,
              min_split_tokens=SPLIT_PLANS[name])
    plan = tw.tw_split_plan(T, **kw)
    assert plan == oracle.split_plan(T, **kw)
    assert plan["reason"] == 0           # the benchmark's step is this split
    prefixes = sorted({T // 2 + off for off in oracle.DEFAULT_OFFSETS} | {plan["prefix_tokens"]})
    for P in prefixes:
        say(f"split {name} prefix={P} suffix={T - P}")
        out, rout = tw.tw_fused_reduce_rmsnorm_split(parts, res, w, d["eps"], P)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(out), out_full)
        np.testing.assert_array_equal(to_host(rout), rout_full)


# --------------------------------------------------- shapes and tails ----

RAGGED = [
    # (N, T, h, dtype): h chosen so the row does not fill the kernel's tiles
    (1, 1, 8, "bf16"), (3, 5, 264, "bf16"), (2, 33, 1032, "bf16"), (5, 7, 2056, "bf16"),
    (8, 9, 4104, "bf16"), (8, 3, 8200, "bf16"), (16, 2, 16392, "bf16"), (4, 2, 24584, "bf16"),
    (2, 3, 65536, "bf16"), (16, 3, 65528, "bf16"),
    (1, 3, 4, "f32"), (2, 17, 516, "f32"), (7, 4, 1028, "f32"), (16, 5, 2052, "f32"),
    (3, 2, 32768, "f32"), (2, 2, 32764, "f32"),
]


@pytest.mark.parametrize("N,T,h,dtype", RAGGED)
def test_ragged_and_extreme_shapes(N, T, h, dtype):
    wl = WORKLOADS["llama70b"] if dtype == "bf16" else WORKLOADS["tiny"]
    d = make_inputs(wl, num_tokens=T, hidden=h)
    d["partials"] = d["partials"][:N] if N <= len(d["partials"]) else np.concatenate(
        [d["partials"]] * (N // len(d["partials"]) + 1))[:N]
    say(f"ragged N={N} T={T} h={h} {dtype}")
    parts, res, w = upload(d)
    out, rout = _run_full(parts, res, w, d["eps"])
    y, x, _ = _oracle(d)
    check(out, y, dtype, "out")
    check(rout, x, dtype, "residual_out")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_closed_form_rows(dtype):
    N, T, h = 3, 66, 1024
    s = special_rows_inputs(N, T, h, dtype)
    parts = to_device(s["partials"], dtype)
    res = to_device(s["residual"], dtype)
    for wkey in ("weight_one", "weight"):
        say(f"closed-form rows {dtype} {wkey}")
        w = to_device(s[wkey], dtype)
        out, rout = _run_full(parts, res, w, 1e-5)
        y, x, _ = oracle.fused_reduce_rmsnorm(list(s["partials"]), s["residual"], s[wkey], 1e-5, dtype)
        check(out, y, dtype, "out")
        check(rout, x, dtype, "residual_out")
        zero = s["kind"] == 0
        assert np.all(out[zero] == 0) and np.all(rout[zero] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_exact_sums_invariants(dtype):
    N, T, h = 8, 40, 8192
    d = integer_scaled_inputs(N, T, h, dtype, kmax=8)
    d["eps"] = 1e-5
    parts, res, w = upload(d)
    say(f"integer-scaled {dtype}: base")
    out, rout = _run_full(parts, res, w, 1e-5)
    y, x, _ = _oracle(d)
    # sums of k/16 are exact, so residual_out is exactly the rounded sum
    want_x = oracle.round_f64_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)
    np.testing.assert_array_equal(rout, want_x)
    check(out, y, dtype, "out")
    say(f"integer-scaled {dtype}: permuted partials")
    perm = [3, 0, 7, 1, 6, 2, 5, 4]
    out_p, rout_p = _run_full([parts[i] for i in perm], res, w, 1e-5)
    np.testing.assert_array_equal(out_p, out)
    np.testing.assert_array_equal(rout_p, rout)
    say(f"integer-scaled {dtype}: negated inputs")
    out_n, rout_n = _run_full(-parts, -res, w, 1e-5)
    # Values compare with +0 == -0: an exactly cancelling sum is +0 under
    # round-to-nearest whatever the signs of its terms, in the oracle too.
    val = oracle.bf16_bits_to_f64 if dtype == "bf16" else (lambda a: a.astype(np.float64))
    np.testing.assert_array_equal(val(out_n), -val(out))
    np.testing.assert_array_equal(val(rout_n), -val(rout))
    say(f"integer-scaled {dtype}: doubled weight")
    out_2, _ = _run_full(parts, res, w * 2, 1e-5)
    dbl = (lambda a: to_host(to_device(a, dtype) * 2))
    np.testing.assert_array_equal(out_2, dbl(out))


def test_in_place_residual_and_nondefault_stream():
    d = make_inputs("llama70b", num_tokens=64, hidden=8192)
    parts, res, w = upload(d)
    say("in-place reference")
    out_ref, rout_ref = _run_full(parts, res, w, d["eps"])
    s = torch.cuda.Stream()
    say("in-place residual on a side stream")
    with torch.cuda.stream(s):
        out, rout = tw.tw_fused_reduce_rmsnorm(parts, res, w, d["eps"], residual_out=res)
    s.synchronize()
    assert rout.data_ptr() == res.data_ptr()
    np.testing.assert_array_equal(to_host(out), out_ref)
    np.testing.assert_array_equal(to_host(res), rout_ref)


def test_empty_and_tiny_batches():
    d = make_inputs("llama70b", num_tokens=3, hidden=512)
    parts, res, w = upload(d)
    out = torch.full_like(res, 7.0)
    say("shard of an empty range (T=3 < N=8, k=0)")
    tw.tw_shard_rmsnorm(parts, res, w, d["eps"], 0, out=out, residual_out=torch.empty_like(res))
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    say("T=0 full mode")
    e = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    o, r = tw.tw_fused_reduce_rmsnorm([e] * 8, e, w, d["eps"])
    assert o.shape == (0, 512)
    say("T=3 full mode")
    out, rout = _run_full(parts, res, w, d["eps"])
    y, x, _ = _oracle(d)
    check(out, y, "bf16", "out")
    check(rout, x, "bf16", "residual_out")


def test_zero_row_with_zero_eps_is_nan_documented():
    # eps = 0 and an all-zero row: 0 * rsqrt(0) = 0 * inf = NaN (documented).
    parts = torch.zeros((1, 2, 64), dtype=torch.float32, device="cuda")
    res = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    res[1] = 1.0
    w = torch.ones(64, dtype=torch.float32, device="cuda")
    say("zero row with eps=0")
    out, _ = tw.tw_fused_reduce_rmsnorm(parts, res, w, 0.0)
    torch.cuda.synchronize()
    assert torch.isnan(out[0]).all() and torch.all(out[1] == 1.0)


# ------------------------------------------------- unfused comparator ----

@pytest.mark.parametrize("name,T,h", [("tiny", 64, 512), ("llama70b", 1024, 8192),
                                      ("mixtral", 512, 4096), ("llama70b", 7, 4104)])
def test_unfused_comparator_matches_its_oracle(name, T, h):
    d = make_inputs(name, num_tokens=T, hidden=h)
    dt = d["dtype"]
    parts, res, w = upload(d)
    say(f"unfused {name}: T={T} h={h} {dt}")
    out, rout, red = tw.tw_unfused_reduce_rmsnorm(parts, res, w, d["eps"])
    torch.cuda.synchronize()
    y, x, red_ref = oracle.unfused_reduce_rmsnorm(list(d["partials"]), d["residual"], d["weight"],
                                                  d["eps"], dt)
    red64 = oracle.bf16_bits_to_f64(red_ref) if dt == "bf16" else red_ref.astype(np.float64)
    n_red = check(to_host(red), red64, dt, "reduced")
    check(to_host(rout), x, dt, "residual_out")
    n_y = check(to_host(out), y, dt, "out")
    say(f"unfused {name}: reduced not bit-exact {n_red}/{red64.size}, out {n_y}/{y.size}")


# --------------------------------------------- fixed number of workgroups ----

# The grid picks the consecutive-rows kernel's form: fewer workgroups than CUs,
# at least one per CU, or a whole round (2500 rows at G = 1251 launch 1250
# workgroups of two rows, more than a round of 512-thread workgroups).
@pytest.mark.parametrize("name,T,h", [("llama70b", 1024, 8192), ("tiny", 64, 512), ("mixtral", 333, 4096),
                                      ("mixtral", 2500, 4096)])
def test_grid_launch_bit_identical_to_one_row_per_workgroup(name, T, h):
    d = make_inputs(name, num_tokens=T, hidden=h)
    parts, res, w = upload(d)
    say(f"grid reference {name}: T={T} h={h}")
    out_ref, rout_ref = _run_full(parts, res, w, d["eps"])
    for G in (1, 2, 3, 8, 100, 256, T // 2 + 1, T - 1, T, T + 5):
        if G < 1:
            continue
        say(f"grid {name}: {G} workgroups")
        out, rout = tw.tw_fused_reduce_rmsnorm_grid(parts, res, w, d["eps"], G)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(out), out_ref)
        np.testing.assert_array_equal(to_host(rout), rout_ref)


# ------------------------------------------------ overlapped layer step ----

def test_overlapped_split_step_equals_one_fused_launch():
    from reduce_rmsnorm_amd.overlap import LayerStep
    T, h, K, N = 300, 1024, 256, 4
    step = LayerStep(T, h, K, N, eps=1e-5, sets=1, seed=3)
    a, b = torch.cuda.current_stream(), torch.cuda.Stream()
    for prefix in (150, 214, 299, 1):
        say(f"overlapped split step T={T} prefix={prefix}")
        step.run_split(0, prefix, a, b)
        a.wait_stream(b)
        torch.cuda.synchronize()
        parts, res, out, rout = step.outputs(0)
        out_s, rout_s = to_host(out), to_host(rout)
        # the same partials (P_0 now holds the GEMM rows) through one launch
        ref_out, ref_rout = _run_full(parts, res, step.weight, 1e-5)
        np.testing.assert_array_equal(out_s, ref_out)
        np.testing.assert_array_equal(rout_s, ref_rout)
    p_host = to_host(parts)
    y, x, _ = oracle.fused_reduce_rmsnorm(list(p_host), to_host(res), to_host(step.weight), 1e-5, "bf16")
    check(out_s, y, "bf16", "out")
    check(rout_s, x, "bf16", "residual_out")
    say("overlapped unsplit step")
    step.run_unsplit(0, a)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(step.outputs(0)[2]), _run_full(parts, res, step.weight, 1e-5)[0])


def test_captured_split_step_replays_match_eager():
    # Graph replays, with eager work and synchronizations between them, must
    # each reproduce the eager step's outputs.
    from reduce_rmsnorm_amd.overlap import LayerStep, capture
    T, h, K, N = 512, 1024, 256, 8
    step = LayerStep(T, h, K, N, eps=1e-5, sets=1, seed=4)
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    say("eager split step (reference)")
    step.run_split(0, 320, a, b)
    a.wait_stream(b)
    torch.cuda.synchronize()
    ref = [to_host(t) for t in step.outputs(0)]
    say("capture split step")
    g = capture(lambda i: step.run_split(i, 320, a, b), a, b, 0)
    for rep in range(4):
        parts, res, out, rout = step.outputs(0)
        out.fill_(0)
        rout.fill_(0)
        parts[0].fill_(0)
        torch.cuda.synchronize()
        say(f"replay {rep}")
        with torch.cuda.stream(a):
            g.replay()
        torch.cuda.synchronize()
        got = [to_host(t) for t in step.outputs(0)]
        for x, y in zip(got, ref):
            np.testing.assert_array_equal(x, y)
        _ = torch.ones(1000, device="cuda").sum().item()      # eager work between replays


def test_graph_replayed_fused_launches_match_eager():
    # The benchmark's graph mode: prepared full, shard and split launches on
    # rotated buffer sets, recorded into one HIP graph on a side stream.  Every
    # replay, with the outputs cleared and eager work in between, must give
    # the eager launches' bits.
    T, h, R = 320, 8192, 3
    d = make_inputs("llama70b", num_tokens=T, hidden=h)
    parts, res, w = upload(d)
    ref_out, ref_rout = _run_full(parts, res, w, d["eps"])
    sets = [(parts.clone(), res.clone(), torch.empty_like(res), torch.empty_like(res))
            for _ in range(R)]
    cap = torch.cuda.Stream()
    P = 192
    launches = []
    for i, (p, r, o, ro) in enumerate(sets):
        if i == 0:
            launches.append(tw.PreparedFused(p, r, w, d["eps"], o, ro, cap))
        elif i == 1:
            launches += [tw.PreparedFused([q[lo:hi] for q in p], r[lo:hi], w, d["eps"], o[lo:hi],
                                          ro[lo:hi], cap) for lo, hi in ((0, P), (P, T))]
        else:
            launches += [tw.PreparedFused(p, r, w, d["eps"], o, ro, cap, mode="shard",
                                          shard_index=k) for k in range(8)]
    say("capture full, split and shard launches into one graph")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for launch in launches:
            launch()
    for rep in range(4):
        for _, _, o, ro in sets:
            o.fill_(float("nan"))
            ro.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for _, _, o, ro in sets:
            np.testing.assert_array_equal(to_host(o), ref_out)
            np.testing.assert_array_equal(to_host(ro), ref_rout)
        _ = torch.ones(1000, device="cuda").sum().item()      # eager work between replays


def test_prepared_launches_match_direct_calls():
    d = make_inputs("llama70b", num_tokens=96, hidden=8192)
    parts, res, w = upload(d)
    ref_out, ref_rout = _run_full(parts, res, w, d["eps"])
    for mode, kw in (("full", {}), ("grid", {"num_workgroups": 7}), ("shard", {"shard_index": 3})):
        out = torch.full_like(res, float("nan"))
        rout = torch.full_like(res, float("nan"))
        say(f"prepared launch, mode {mode}")
        launch = tw.PreparedFused(parts, res, w, d["eps"], out, rout, mode=mode, **kw)
        launch()
        launch()
        torch.cuda.synchronize()
        rows = oracle.shard_rows(96, 8, 3) if mode == "shard" else range(96)
        sl = slice(rows.start, rows.stop)
        np.testing.assert_array_equal(to_host(out)[sl], ref_out[sl])
        np.testing.assert_array_equal(to_host(rout)[sl], ref_rout[sl])
    cache = tw.SplitPlanCache(tokens_per_cta=256, ctas_per_token_tile=32, num_cus=256,
                              min_split_tokens=1024)
    assert cache(4096) == oracle.split_plan(4096, tokens_per_cta=256, ctas_per_token_tile=32,
                                            num_cus=256, min_split_tokens=1024)
    plan = cache(4096)
    plan["offset"] = 99
    assert cache(4096)["offset"] == 0                      # cached plans are handed out as copies


@pytest.mark.parametrize("N", list(range(1, 17)))
def test_every_partial_count_at_the_headline_width(N):
    d = make_inputs("llama70b", num_tokens=12, hidden=8192, seed=100 + N)
    d["partials"] = np.concatenate([d["partials"]] * 2)[:N]
    parts, res, w = upload(d)
    say(f"N={N} T=12 h=8192 (full and 5-workgroup grid)")
    out, rout = _run_full(parts, res, w, d["eps"])
    y, x, _ = _oracle(d)
    check(out, y, "bf16", "out")
    check(rout, x, "bf16", "residual_out")
    o2, r2 = tw.tw_fused_reduce_rmsnorm_grid(parts, res, w, d["eps"], 5)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(o2), out)
    np.testing.assert_array_equal(to_host(r2), rout)


def test_pointer_checks_reject_host_memory():
    d = make_inputs("llama70b", num_tokens=16, hidden=1024)
    parts, res, w = upload(d)
    host_part = torch.empty((16, 1024), dtype=torch.bfloat16, pin_memory=True)
    host_part.copy_(parts[0].cpu())
    tw.tw_set_pointer_checks(True)
    try:
        say("pointer checks on: device tensors pass")
        out, _ = tw.tw_fused_reduce_rmsnorm(parts, res, w, d["eps"])
        torch.cuda.synchronize()
        say("pointer checks on: a pinned host partial is rejected before launch")
        lib = tw.load_library()
        import ctypes
        ptrs = (ctypes.c_void_p * 2)(host_part.data_ptr(), parts[1].data_ptr())
        o = torch.empty_like(res)
        r = torch.empty_like(res)
        st = lib.tw_fused_reduce_rmsnorm(ptrs, 2, res.data_ptr(), w.data_ptr(), o.data_ptr(),
                                         r.data_ptr(), 16, 1024, ctypes.c_float(1e-5), 1, None)
        assert st == 1 and b"not device memory" in lib.tw_last_error()
    finally:
        tw.tw_set_pointer_checks(False)
    ref, _ = _run_full(parts, res, w, d["eps"])
    np.testing.assert_array_equal(to_host(out), ref)


def test_nan_input_propagates_to_its_row_only():
    # NaN and inf are outside the contract; the documented behaviour is that
    # they propagate: a NaN in one row makes that row's outputs NaN (its sum
    # of squares is NaN) and leaves every other row exact.
    d = make_inputs("llama70b", num_tokens=6, hidden=4096)
    d["partials"] = d["partials"].copy()
    d["partials"][2, 3, 100] = 0x7FC0          # quiet NaN in row 3
    parts, res, w = upload(d)
    say("NaN in one partial element")
    out, rout = _run_full(parts, res, w, d["eps"])
    val = oracle.bf16_bits_to_f64(out)
    assert np.isnan(val[3]).all()
    rval = oracle.bf16_bits_to_f64(rout)
    assert np.isnan(rval[3, 100]) and np.isfinite(np.delete(rval[3], 100)).all()
    keep = [0, 1, 2, 4, 5]
    y, x, _ = _oracle(d, rows=keep)
    check(out[keep], y, "bf16", "out")
    check(rout[keep], x, "bf16", "residual_out")


@pytest.mark.parametrize("num_cus,T,kernel", [(8, 200, "seq"), (64, 150, "all"),
                                              (64, 200, "seq"), (64, 296, "strided"),
                                              (256, 200, "all")])
def test_cu_masked_stream_matches_oracle_and_takes_its_own_round(num_cus, T, kernel):
    # The first k mask bits spread k CUs evenly over the XCDs (bit b belongs to
    # XCD b mod 8).  The launch rules size a round from the CUs the stream may
    # use: on 64 CUs a round of 1024-thread workgroups is 128 rows, so 150 rows
    # (just past one round, N = 8) issue all loads at once, 200 rows load in
    # sequence and 296 rows (a last round of 40) run the strided kernel, where
    # the whole device would issue all loads at once for each.  Where the
    # workgroups run must not change a single bit, and every row must meet
    # the oracle.
    from reduce_rmsnorm_amd.overlap import MaskedStream, mask_words
    d = make_inputs("llama70b", num_tokens=T, hidden=8192, seed=7)
    parts, res, w = upload(d)
    ref_out, ref_rout = _run_full(parts, res, w, d["eps"])
    say(f"fused launch of {T} rows on a stream masked to {num_cus} CUs")
    with MaskedStream(range(num_cus)) as ms:
        assert ms.mask() == mask_words(range(num_cus))
        info = tw.tw_fused_launch_info(8, T, 8192, stream=ms.stream)
        assert (info["num_cus"], info["round_rows"], info["kernel_name"]) == \
            (num_cus, 2 * num_cus, kernel), info
        out = torch.full_like(res, float("nan"))
        rout = torch.full_like(res, float("nan"))
        tw.PreparedFused(parts, res, w, d["eps"], out, rout, ms.stream)()
        ms.stream.synchronize()
    np.testing.assert_array_equal(to_host(out), ref_out)
    np.testing.assert_array_equal(to_host(rout), ref_rout)
    y, x, _ = _oracle(d)
    check(ref_out, y, "bf16", "out")
    check(ref_rout, x, "bf16", "residual_out")


def test_device_cu_count_sizes_the_round():
    # The null stream and a plain stream may use every CU of the device.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for st in (None, torch.cuda.Stream()):
        info = tw.tw_fused_launch_info(8, 1024, 8192, stream=st)
        assert info["num_cus"] == cus and info["round_rows"] == 2 * cus, info


def test_row_count_beyond_one_dispatch():
    # 70 M rows of 8 bf16 elements run 64-thread workgroups: 4.5e9 work-items,
    # more than one dispatch carries (below 2^31).  The fused launch, whose
    # dispatches also stay within 768 MiB of traffic, takes seven dispatches
    # of 10 M rows; the unfused kernels take three over consecutive row
    # ranges; the consecutive-rows kernel asked for 69 M workgroups (35 M of
    # them holding two rows, 2.2e9 work-items) is capped to 33.5 M workgroups
    # of three rows.  Every row must still be computed, once, with the same
    # bits, on both sides of every dispatch boundary.
    T, h, N = 70_000_000, 8, 2
    chunk = (2 ** 31 - 1) // 64
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    parts = (torch.randn(N, T, h, device="cuda", generator=g, dtype=torch.bfloat16) * 0.5)
    res = torch.randn(T, h, device="cuda", generator=g, dtype=torch.bfloat16)
    w = (1 + 0.05 * torch.randn(h, device="cuda", generator=g)).to(torch.bfloat16)
    eps = 1e-5
    say(f"fused, T={T} h={h} N={N}: more rows than one dispatch holds")
    out, rout = tw.tw_fused_reduce_rmsnorm(parts, res, w, eps)
    say("grid launch asking for 69 M workgroups")
    out_g, rout_g = tw.tw_fused_reduce_rmsnorm_grid(parts, res, w, eps, 69_000_000)
    torch.cuda.synchronize()
    assert torch.equal(out_g, out) and torch.equal(rout_g, rout)
    del out_g, rout_g
    say("unfused comparator on the same rows")
    out_u, rout_u, _ = tw.tw_unfused_reduce_rmsnorm(parts, res, w, eps)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    idx = np.unique(np.concatenate([
        np.arange(4), np.arange(chunk - 3, chunk + 3), np.arange(2 * chunk - 3, 2 * chunk + 3),
        *[np.arange(k * 10_000_000 - 3, k * 10_000_000 + 3) for k in range(1, 7)],
        np.arange(T - 4, T), rng.integers(0, T, 4000)]))
    ti = torch.from_numpy(idx).to("cuda")
    p_host = [to_host(parts[i].index_select(0, ti)) for i in range(N)]
    r_host = to_host(res.index_select(0, ti))
    y, x, _ = oracle.fused_reduce_rmsnorm(p_host, r_host, to_host(w), eps, "bf16")
    check(to_host(out.index_select(0, ti)), y, "bf16", "out")
    check(to_host(rout.index_select(0, ti)), x, "bf16", "residual_out")
    yu, xu, _ = oracle.unfused_reduce_rmsnorm(p_host, r_host, to_host(w), eps, "bf16")
    check(to_host(out_u.index_select(0, ti)), yu, "bf16", "unfused out")
    check(to_host(rout_u.index_select(0, ti)), xu, "bf16", "unfused residual_out")


def test_long_call_cut_into_dispatches():
    # 8193 rows of h = 8192 with N = 8 move 1.48 GB, more than one dispatch
    # may (768 MiB): the call runs as three dispatches of 2731 rows.  Rows on
    # both sides of each boundary match the oracle, and every row matches the
    # grid launch, whose dispatches are laid out differently.
    T, h, N = 8193, 8192, 8
    d = make_inputs("llama70b", num_tokens=T, hidden=h)
    parts, res, w = upload(d)
    say(f"fused, T={T} h={h} N={N}: three dispatches")
    out, rout = tw.tw_fused_reduce_rmsnorm(parts, res, w, d["eps"])
    say("grid launch over the same rows")
    out_g, rout_g = tw.tw_fused_reduce_rmsnorm_grid(parts, res, w, d["eps"], 700)
    torch.cuda.synchronize()
    assert torch.equal(out_g, out) and torch.equal(rout_g, rout)
    rows = np.unique(np.concatenate([np.arange(0, 3), np.arange(2729, 2734),
                                     np.arange(5460, 5465), np.arange(T - 3, T)]))
    y, x, _ = oracle.fused_reduce_rmsnorm([p[rows] for p in d["partials"]], d["residual"][rows],
                                          d["weight"], d["eps"], "bf16")
    check(to_host(out)[rows], y, "bf16", "out")
    check(to_host(rout)[rows], x, "bf16", "residual_out")


def test_random_shapes_match_oracle():
    # Seeded random shapes across the supported range: N in 1..16, T in
    # 1..70, row widths from one 16-byte vector to the largest row (around
    # every geometry boundary), both dtypes, eps 1e-6 to 1e-2.  Every
    # third case also runs shard k and a grid launch, which must give the
    # same bits on their rows.
    rng = np.random.default_rng(2024)
    for case in range(60):
        dtype = "bf16" if rng.random() < 0.6 else "f32"
        per_vec = 8 if dtype == "bf16" else 4
        max_vec = (65536 if dtype == "bf16" else 32768) // per_vec
        nvec = int(rng.choice([1, 2, 3, 7, 31, 64, 127, 256, 511, 512, 513, 1023, 1024, 1025,
                               2047, 2048, 2049, 4095, 4096, max_vec - 1, max_vec]))
        h = nvec * per_vec
        N = int(rng.integers(1, 17))
        T = int(rng.integers(1, 71)) if h <= 16384 else int(rng.integers(1, 9))
        eps = float(rng.choice([1e-6, 1e-5, 1e-2]))
        wl = WORKLOADS["llama70b"] if dtype == "bf16" else WORKLOADS["tiny"]
        d = make_inputs(wl, num_tokens=T, hidden=h, seed=1000 + case)
        d["partials"] = np.concatenate([d["partials"]] * (N // len(d["partials"]) + 1))[:N]
        d["eps"] = eps
        say(f"random case {case}: N={N} T={T} h={h} {dtype} eps={eps}")
        parts, res, w = upload(d)
        out, rout = _run_full(parts, res, w, eps)
        y, x, _ = _oracle(d)
        check(out, y, dtype, f"case {case} out")
        check(rout, x, dtype, f"case {case} residual_out")
        if case % 3 == 0:
            k = int(rng.integers(0, N))
            lo, hi = oracle.shard_rows(T, N, k).start, oracle.shard_rows(T, N, k).stop
            o_s, r_s = torch.zeros_like(res), torch.zeros_like(res)
            tw.tw_shard_rmsnorm(parts, res, w, eps, k, out=o_s, residual_out=r_s)
            o_g, r_g = tw.tw_fused_reduce_rmsnorm_grid(parts, res, w, eps,
                                                       int(rng.integers(1, T + 1)))
            torch.cuda.synchronize()
            np.testing.assert_array_equal(to_host(o_s)[lo:hi], out[lo:hi])
            np.testing.assert_array_equal(to_host(r_s)[lo:hi], rout[lo:hi])
            np.testing.assert_array_equal(to_host(o_g), out)
            np.testing.assert_array_equal(to_host(r_g), rout)


def test_binding_rejects_mismatched_tensors():
    d = make_inputs("llama70b", num_tokens=8, hidden=256)
    parts, res, w = upload(d)
    say("binding argument checks")
    bad = [
        (lambda: tw.tw_fused_reduce_rmsnorm(parts, res.float(), w, 1e-5), "dtype"),
        (lambda: tw.tw_fused_reduce_rmsnorm(parts[:, :4], res, w, 1e-5), "shape"),
        (lambda: tw.tw_fused_reduce_rmsnorm(parts, res, w[:128], 1e-5), "weight"),
        (lambda: tw.tw_fused_reduce_rmsnorm(parts, res.t().contiguous().t(), w, 1e-5),
         "contiguous"),
        (lambda: tw.tw_fused_reduce_rmsnorm(parts, res, w, 1e-5, out=torch.empty(8, 128, dtype=res.dtype,
                                                                                  device="cuda")),
         "out"),
        (lambda: tw.tw_fused_reduce_rmsnorm(parts, res, w.cpu(), 1e-5), "GPU"),
        (lambda: tw.PreparedFused(parts, res, w, 1e-5, torch.empty_like(res),
                                  torch.empty_like(res), mode="rows"), "mode"),
    ]
    for fn, needle in bad:
        with pytest.raises(ValueError, match=needle):
            fn()
    # Errors the library itself finds come back as TokenWeaveError with its text.
    with pytest.raises(tw.TokenWeaveError, match="eps"):
        tw.tw_fused_reduce_rmsnorm(parts, res, w, float("nan"))
    with pytest.raises(tw.TokenWeaveError, match="shard_index"):
        tw.tw_shard_rmsnorm(parts, res, w, 1e-5, shard_index=len(parts))


def test_row_whose_sum_of_squares_overflows_float32():
    # x = 2^70 in every element: x^2 = 2^140 overflows float32, so rs = 0 and
    # the documented result is out = 0 for that row, residual_out = x exactly.
    # The neighbouring rows are untouched by it.
    d = make_inputs("llama70b", num_tokens=3, hidden=512)
    big = np.uint16(0x6280)          # bf16 bits of 2^70
    d["partials"][:, 1, :] = 0
    d["partials"][0, 1, :] = big
    d["residual"][1, :] = 0
    parts, res, w = upload(d)
    say("row with x = 2^70: float32 sum of squares overflows")
    out, rout = _run_full(parts, res, w, d["eps"])
    assert oracle.bf16_bits_to_f64(np.array([big]))[0] == 2.0 ** 70
    assert (out[1] & 0x7FFF == 0).all(), "out of the overflowing row must be +-0"
    np.testing.assert_array_equal(rout[1], np.full(512, big))
    y, x, _ = _oracle(d, rows=[0, 2])
    check(out[[0, 2]], y, "bf16", "out, other rows")
    check(rout[[0, 2]], x, "bf16", "residual_out, other rows")


@pytest.mark.parametrize("h,N,dtype,T", [(8192, 5, "bf16", 1100), (8192, 6, "bf16", 1100),
                                         (8192, 8, "bf16", 1100), (8192, 16, "bf16", 1100),
                                         (4096, 2, "bf16", 1100), (4096, 8, "bf16", 1600),
                                         (8184, 8, "bf16", 1100), (12296, 3, "bf16", 1100),
                                         (16384, 8, "bf16", 1100), (3080, 4, "bf16", 1100),
                                         (4096, 8, "f32", 1100), (2048, 3, "f32", 1100),
                                         (8192, 2, "f32", 1100), (4092, 7, "f32", 1100),
                                         (5120, 8, "bf16", 1600), (5112, 16, "bf16", 1600),
                                         (2560, 8, "bf16", 3200), (2552, 12, "bf16", 3200),
                                         (3072, 2, "bf16", 1400), (1280, 4, "f32", 3100),
                                         (12288, 8, "bf16", 2200), (12280, 16, "bf16", 2200),
                                         (2560, 1, "bf16", 1100), (1536, 1, "f32", 1100),
                                         (16384, 8, "bf16", 2048)])
def test_load_order_never_changes_a_bit(h, N, dtype, T):
    # A launch that fills every CU loads the tensors in summation order; a
    # smaller one (here each of the N shards) issues all loads at once.  The
    # arithmetic is the same, so every row must come out bit-identical, and
    # both must meet the oracle.
    # T is above one full round of workgroups at every width here (512 rows
    # for the 1024-thread classes, 1024 rows for 512 x 1) and past the window
    # just above one round where launches with a long sequence per thread
    # issue all loads at once (hence 1600 rows for h = 4096, N = 8).  Where
    # the last round is at most half full the full launch takes the strided
    # kernel (not h = 16384 or 12296 bf16, nor 8192 f32); the ragged widths
    # (8184, 12296, 3080) leave lanes that clamp their address inside the
    # sequence.  h = 5120 (N >= 7), 2560, 3072 and f32 1280 run the 640-, 320-
    # and 384-thread workgroups (rounds of 768, 1536 and 1280 rows), 5112 and
    # 2552 with a lane that clamps; 12288 and 12280 run 512 x 3, whose short
    # form (the shards) keeps three tensors in flight per vector slot.  With
    # one partial the 320- and 384-thread classes issue all loads at once in
    # every launch (N = 1 has no sequenced order).
    d = make_inputs("llama70b" if dtype == "bf16" else "tiny", num_tokens=T, hidden=h, seed=40 + N)
    # N partials: the drawn ones, then copies with their rows in reverse order.
    d["partials"] = np.concatenate([d["partials"]] + [d["partials"][:, ::-1]] * 8)[:N]
    parts, res, w = upload(d)
    say(f"load orders: T={T} h={h} N={N} {dtype}")
    out, rout = _run_full(parts, res, w, d["eps"])
    out_s = torch.full_like(res, float("nan"))
    rout_s = torch.full_like(res, float("nan"))
    for k in range(N):
        tw.tw_shard_rmsnorm(parts, res, w, d["eps"], shard_index=k, out=out_s, residual_out=rout_s)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(out_s), out)
    np.testing.assert_array_equal(to_host(rout_s), rout)
    rows = list(range(0, T, 37))
    y, x, _ = _oracle(d, rows=rows)
    check(out[rows], y, dtype, "out")
    check(rout[rows], x, dtype, "residual_out")


@pytest.mark.parametrize("h,N,T", [(16384, 8, 256), (16384, 4, 240), (16384, 11, 250),
                                   (12288, 4, 256), (16376, 8, 256)])
def test_both_slots_launch_matches_one_slot_launches_and_oracle(h, N, T):
    # A launch that gives nearly every CU one workgroup of 1024 x 2 loads
    # both vector slots at once; the same rows as two launches of half the
    # rows each load one slot at a time.  Same bits, and every sampled row
    # meets the oracle (16376 leaves lanes that clamp their address).
    info = tw.tw_fused_launch_info(N, T, h)
    cus = info["num_cus"]
    if not (8 * T > 7 * cus and T <= cus):
        pytest.skip(f"{T} rows do not give each of {cus} CUs one workgroup")
    assert info["kernel_name"] == "both" and tw.tw_fused_launch_info(N, T // 2, h)["kernel_name"] == "all"
    d = make_inputs("llama405b", num_tokens=T, hidden=h, seed=90 + N)
    d["partials"] = np.concatenate([d["partials"]] + [d["partials"][:, ::-1]] * 2)[:N]
    parts, res, w = upload(d)
    say(f"both slots at once: T={T} h={h} N={N}")
    out, rout = _run_full(parts, res, w, d["eps"])
    out_p = torch.full_like(res, float("nan"))
    rout_p = torch.full_like(res, float("nan"))
    for lo, hi in ((0, T // 2), (T // 2, T)):
        tw.tw_fused_reduce_rmsnorm(parts[:, lo:hi], res[lo:hi], w, d["eps"], out=out_p[lo:hi],
                                   residual_out=rout_p[lo:hi])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(out_p), out)
    np.testing.assert_array_equal(to_host(rout_p), rout)
    rows = sorted(set(range(0, T, 17)) | {T - 1})
    y, x, _ = _oracle(d, rows=rows)
    check(out[rows], y, "bf16", "out")
    check(rout[rows], x, "bf16", "residual_out")


# Launches whose row count is not a whole number of rounds (a round: 512
# workgroups for the 1024-thread classes, h = 8192 or 16384 bf16 and 4096 or
# 8192 f32; 1024 for 512 x 1, h = 4096 bf16).  The first nine cases have a
# last round at most half full within four rounds and run the strided kernel
# (N = 5 loads two tensors ahead, the others one; 8184 and 4088 leave lanes
# that clamp their address).  The other seven lie between one and one and a
# half rounds with at least 8 tensors in each thread's sequence, and issue all
# loads at once; of the last three, two run the 640- and 320-thread
# workgroups (rounds of 768 and 1536 rows) and one 512 x 3 (1024 rows, its
# short form keeping three tensors in flight).
RAGGED_ROUNDS = [(8192, 8, "bf16", 768), (8192, 5, "bf16", 600), (8192, 16, "bf16", 1280),
           (8184, 7, "bf16", 1200), (4096, 8, "bf16", 1536), (4096, 2, "bf16", 1536),
           (4088, 3, "bf16", 1100), (4096, 8, "f32", 1100), (4096, 12, "f32", 1700),
           (8192, 8, "bf16", 600), (8184, 16, "bf16", 544), (4096, 8, "bf16", 1100),
           (16384, 8, "bf16", 576), (8192, 7, "f32", 600),
           (5120, 16, "bf16", 800), (2560, 8, "bf16", 1700), (12288, 8, "bf16", 1100)]


def _round_rows(h, elem_bytes, n):
    """Rows one round of resident workgroups holds on this device, for the
    sequenced row classes these tests use: 2048 threads per CU divided among
    the row class's workgroups (the fitted 320-, 384- and 640-thread classes
    and 512 x 3 included), as the library counts it."""
    info = tw.tw_fused_launch_info(n, 1, h, torch.bfloat16 if elem_bytes == 2 else torch.float32)
    assert info["round_rows"] == info["num_cus"] * (2048 // info["threads_per_workgroup"])
    return info["round_rows"]


@pytest.mark.parametrize("h,N,dtype,T", RAGGED_ROUNDS)
def test_ragged_round_launch_matches_whole_round_launches_and_oracle(h, N, dtype, T):
    d = make_inputs("llama70b" if dtype == "bf16" else "tiny", num_tokens=T, hidden=h, seed=70 + N)
    d["partials"] = np.concatenate([d["partials"]] + [d["partials"][:, ::-1]] * 8)[:N]
    parts, res, w = upload(d)
    round_rows = _round_rows(h, 2 if dtype == "bf16" else 4, N)
    whole = (T // round_rows) * round_rows
    say(f"ragged rounds: T={T} h={h} N={N} {dtype}; pieces [0,{whole}) and [{whole},{T})")
    out = torch.full_like(res, float("nan"))
    rout = torch.full_like(res, float("nan"))
    tw.tw_fused_reduce_rmsnorm(parts, res, w, d["eps"], out=out, residual_out=rout)
    # The same rows as whole rounds of one-row workgroups, loaded in sequence,
    # plus the remainder, which is under one round and issues all loads at once.
    out_p = torch.full_like(res, float("nan"))
    rout_p = torch.full_like(res, float("nan"))
    for lo, hi in ((0, whole), (whole, T)):
        tw.tw_fused_reduce_rmsnorm(parts[:, lo:hi], res[lo:hi], w, d["eps"], out=out_p[lo:hi],
                                   residual_out=rout_p[lo:hi])
    torch.cuda.synchronize()
    o, ro = to_host(out), to_host(rout)
    np.testing.assert_array_equal(to_host(out_p), o)
    np.testing.assert_array_equal(to_host(rout_p), ro)
    rows = sorted(set(range(0, T, 23)) | {T - 1, whole - 1, whole})
    y, x, _ = _oracle(d, rows=rows)
    check(o[rows], y, dtype, "out")
    check(ro[rows], x, dtype, "residual_out")


@pytest.mark.parametrize("h,N,T", [(8192, 16, 3300), (16384, 16, 2100)])
def test_each_dispatch_of_a_long_call_takes_its_own_kernel(h, N, T):
    # A call over 768 MiB of traffic is cut into dispatches of about equal
    # size, each a launch of its own: 2 x 1650 rows at h = 8192 (the strided
    # kernel) and 3 x 700 rows at h = 16384 (all loads at once, being between
    # one and one and a half rounds), with 16 partials.  Bit for bit against
    # one launch per shard (all loads at once), and sampled rows, on both
    # sides of every dispatch boundary, against the oracle.
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    parts = (torch.randn(N, T, h, device="cuda", generator=g, dtype=torch.bfloat16) * 0.5)
    res = torch.randn(T, h, device="cuda", generator=g, dtype=torch.bfloat16)
    w = (1 + 0.05 * torch.randn(h, device="cuda", generator=g)).to(torch.bfloat16)
    eps = 1e-5
    say(f"long call: T={T} h={h} N={N}")
    out, rout = tw.tw_fused_reduce_rmsnorm(parts, res, w, eps)
    out_s = torch.full_like(res, float("nan"))
    rout_s = torch.full_like(res, float("nan"))
    for k in range(N):
        tw.tw_shard_rmsnorm(parts, res, w, eps, shard_index=k, out=out_s, residual_out=rout_s)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out) and torch.equal(rout_s, rout)
    piece = 1650 if h == 8192 else 700
    idx = np.unique(np.concatenate([np.arange(0, T, 97), np.arange(T - 3, T)] +
                                   [np.arange(b - 3, b + 3) for b in range(piece, T, piece)]))
    ti = torch.from_numpy(idx).to("cuda")
    y, x, _ = oracle.fused_reduce_rmsnorm([to_host(parts[i].index_select(0, ti)) for i in range(N)],
                                          to_host(res.index_select(0, ti)), to_host(w), eps, "bf16")
    check(to_host(out.index_select(0, ti)), y, "bf16", "out")
    check(to_host(rout.index_select(0, ti)), x, "bf16", "residual_out")


@pytest.mark.parametrize("eps", [0.0, 1e-12, 1e-5, 1.0])
def test_subnormal_tiny_and_huge_rows_with_extreme_eps(eps):
    # Row 0: subnormal bf16 inputs (float32 subnormals once widened), where
    # float32 squares underflow to zero; row 1: tiny normal values (~1e-30,
    # squares underflow); row 2: large values (~1e17, squares near the top of
    # float32); row 3: ordinary values.  eps = 0 is left out for rows whose
    # sum of squares underflows to zero in float32 (0/0 is the documented NaN).
    rng = np.random.default_rng(77)
    d = make_inputs("llama70b", num_tokens=4, hidden=512, seed=77)
    sign = lambda shape: (rng.integers(0, 2, shape).astype(np.uint16) << 15)
    d["partials"][:, 0, :] = sign((8, 512)) | rng.integers(1, 0x80, (8, 512)).astype(np.uint16)
    d["residual"][0, :] = sign(512) | rng.integers(1, 0x80, 512).astype(np.uint16)
    tiny = oracle.round_f64_to_bf16_bits(rng.normal(0, 1e-30, (8, 512)))
    d["partials"][:, 1, :] = tiny
    d["residual"][1, :] = oracle.round_f64_to_bf16_bits(rng.normal(0, 1e-30, 512))
    d["partials"][:, 2, :] = oracle.round_f64_to_bf16_bits(rng.normal(0, 1e17, (8, 512)))
    d["residual"][2, :] = oracle.round_f64_to_bf16_bits(rng.normal(0, 1e17, 512))
    parts, res, w = upload(d)
    say(f"subnormal / tiny / huge rows, eps={eps}")
    out, rout = _run_full(parts, res, w, eps)
    rows = [0, 1, 2, 3] if eps > 0 else [2, 3]
    d["eps"] = eps
    y, x, _ = _oracle(d, rows=rows)
    check(rout[rows], x, "bf16", "residual_out")
    check(out[rows], y, "bf16", "out")


@pytest.mark.parametrize("N,T,h", [(12, 600, 8192), (16, 1100, 4096), (16, 520, 16384), (3, 40, 8192),
                                   (8, 1700, 2560), (2, 1400, 3072), (8, 900, 5120), (8, 1300, 12288),
                                   (16, 200, 12280)])
def test_unfused_comparator_many_partials(N, T, h):
    # The comparator's reduce step uses the fused geometry and load orders
    # (sequenced above one full round of workgroups), with no occupancy cap
    # above ten partials; its add + RMSNorm step takes the row class's base
    # workgroup, which for h = 2560, 3072, 5120 and 12288 is the fitted one
    # (320, 384, 640 threads, 512 x 3).
    d = make_inputs("llama70b", num_tokens=T, hidden=h, seed=60 + N)
    d["partials"] = np.concatenate([d["partials"], d["partials"][:, ::-1]])[:N]
    parts, res, w = upload(d)
    say(f"unfused comparator N={N} T={T} h={h}")
    out, rout, red = tw.tw_unfused_reduce_rmsnorm(parts, res, w, d["eps"])
    torch.cuda.synchronize()
    rows = list(range(0, T, 29))
    y, x, red_ref = oracle.unfused_reduce_rmsnorm([p[rows] for p in d["partials"]], d["residual"][rows],
                                                  d["weight"], d["eps"], "bf16")
    check(to_host(red)[rows], oracle.bf16_bits_to_f64(red_ref), "bf16", "reduced")
    check(to_host(rout)[rows], x, "bf16", "residual_out")
    check(to_host(out)[rows], y, "bf16", "out")
