"""C-ABI tests that need no GPU: the library loads, exports every function
the header declares, rejects every invalid argument before touching the
device, and its split planner matches the oracle bit for bit.

No call here reaches a kernel launch: each fused/shard call carries at least
one invalid argument, or num_tokens == 0 (a documented no-op)."""

import ctypes
import os
import re
import random
import subprocess

import pytest

import oracle
import reduce_rmsnorm_amd as tw
from reduce_rmsnorm_amd import _lib

INVALID, UNSUPPORTED = _lib.TW_ERR_INVALID_ARG, _lib.TW_ERR_UNSUPPORTED


@pytest.fixture(scope="module")
def lib():
    return tw.load_library()


def test_exports_every_declared_symbol(lib):
    names = tw.declared_functions()
    assert set(names) >= {"tw_fused_reduce_rmsnorm", "tw_shard_rmsnorm", "tw_split_plan",
                          "tw_status_string", "tw_last_error", "tw_abi_version"}
    for n in names:
        assert hasattr(lib, n), n
    dyn = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in dyn.splitlines() if " T " in ln}
    assert set(names) <= exported
    header = open(tw.declared_functions.__defaults__[0]).read()
    assert lib.tw_abi_version() == int(re.search(r"#define TW_ABI_VERSION (\d+)", header).group(1))


def test_every_entry_point_has_a_python_binding():
    support = {"tw_status_string", "tw_last_error", "tw_abi_version"}
    for n in tw.declared_functions():
        if n not in support:
            assert callable(getattr(tw, n, None)), f"reduce_rmsnorm_amd.{n} missing"


def test_status_strings(lib):
    for s in range(4):
        assert lib.tw_status_string(s).startswith(b"TW_")
    assert lib.tw_status_string(99) == b"unknown tw_status"


# ------------------------------------------------------------ validation ----

A = 0x7F0000000000          # fake, 16-byte aligned "device" addresses (never dereferenced)
MB = 1 << 20


def _call(lib, n=2, T=4, h=64, eps=1e-5, dtype=1, parts=None, res=A + 10 * MB, w=A + 11 * MB,
          out=A + 12 * MB, rout=A + 13 * MB, shard=None):
    if parts is None:
        parts = [A + i * MB for i in range(n)]
    arr = (ctypes.c_void_p * max(1, len(parts)))(*parts) if parts is not False else None
    args = [arr, n, res, w, out, rout, T, h, ctypes.c_float(eps), dtype]
    if shard is None:
        return lib.tw_fused_reduce_rmsnorm(*args, None)
    return lib.tw_shard_rmsnorm(*args, shard, None)


@pytest.mark.parametrize("shard", [None, 0])
@pytest.mark.parametrize("kw,code,needle", [
    (dict(n=0, parts=[A]), INVALID, "num_partials"),
    (dict(n=17, parts=[A + i * MB for i in range(17)]), INVALID, "num_partials"),
    (dict(T=-1), INVALID, "num_tokens"),
    (dict(h=0), INVALID, "hidden"),
    (dict(eps=-1e-5), INVALID, "eps"),
    (dict(eps=float("inf")), INVALID, "eps"),
    (dict(eps=float("nan")), INVALID, "eps"),
    (dict(dtype=7), INVALID, "dtype"),
    (dict(h=12), UNSUPPORTED, "multiple"),              # bf16 needs h % 8 == 0
    (dict(h=6, dtype=0), UNSUPPORTED, "multiple"),      # fp32 needs h % 4 == 0
    (dict(h=65544), UNSUPPORTED, "exceeds"),
    (dict(h=32772, dtype=0), UNSUPPORTED, "exceeds"),
    (dict(h=2 ** 62 + 4), UNSUPPORTED, "exceeds"),      # h * 2 would overflow int64
    (dict(h=2 ** 63 - 1, dtype=0), UNSUPPORTED, "exceeds"),
    (dict(T=2 ** 31), UNSUPPORTED, "exceeds"),
    (dict(parts=False), INVALID, "partials array is NULL"),
    (dict(parts=[A, 0]), INVALID, "partials[1] is NULL"),
    (dict(res=0), INVALID, "residual is NULL"),
    (dict(w=0), INVALID, "weight is NULL"),
    (dict(out=0), INVALID, "out is NULL"),
    (dict(rout=0), INVALID, "residual_out is NULL"),
    (dict(parts=[A, A + MB + 8]), UNSUPPORTED, "partials[1] is not 16-byte aligned"),
    (dict(res=A + 10 * MB + 4), UNSUPPORTED, "residual is not 16-byte aligned"),
    (dict(w=A + 11 * MB + 2), UNSUPPORTED, "weight is not 16-byte aligned"),
    (dict(out=A + 12 * MB + 8), UNSUPPORTED, "out is not 16-byte aligned"),
    (dict(rout=A + 13 * MB + 8), UNSUPPORTED, "residual_out is not 16-byte aligned"),
    (dict(out=A + 13 * MB + 16), INVALID, "out overlaps residual_out"),
    (dict(out=A), INVALID, "out overlaps partials[0]"),
    (dict(out=A + 10 * MB + 256), INVALID, "out overlaps residual"),
    (dict(out=A + 11 * MB), INVALID, "out overlaps weight"),
    (dict(rout=A + MB), INVALID, "residual_out overlaps partials[1]"),
    (dict(rout=A + 10 * MB + 16), INVALID, "residual_out overlaps residual"),
    (dict(rout=A + 11 * MB - 16), INVALID, "residual_out overlaps weight"),
])
def test_invalid_arguments_rejected_before_any_device_call(lib, kw, code, needle, shard):
    assert _call(lib, shard=shard, **kw) == code
    assert needle in lib.tw_last_error().decode()


def test_unfused_entries_validate(lib):
    arr = (ctypes.c_void_p * 2)(A, A + MB)
    assert lib.tw_reduce_partials(arr, 0, A + 12 * MB, 4, 64, 1, None) == INVALID
    assert lib.tw_reduce_partials(arr, 2, None, 4, 64, 1, None) == INVALID
    assert lib.tw_reduce_partials(arr, 2, A + 16, 4, 64, 1, None) == INVALID     # overlaps partial 0
    assert b"reduced overlaps partials[0]" in lib.tw_last_error()
    assert lib.tw_reduce_partials(arr, 2, A + 12 * MB + 8, 4, 64, 1, None) == UNSUPPORTED
    assert lib.tw_reduce_partials(arr, 2, A + 12 * MB, 4, 12, 1, None) == UNSUPPORTED
    assert lib.tw_reduce_partials(None, 2, None, 0, 64, 1, None) == 0           # T == 0: no-op
    args = [A, A + 10 * MB, A + 11 * MB, A + 12 * MB, A + 13 * MB, 4, 64]
    assert lib.tw_add_rmsnorm(*args, ctypes.c_float(-1.0), 1, None) == INVALID
    assert lib.tw_add_rmsnorm(A, A + 10 * MB, A + 11 * MB, A, A + 13 * MB, 4, 64,
                              ctypes.c_float(1e-5), 1, None) == INVALID          # out == input
    assert b"out overlaps input" in lib.tw_last_error()
    # residual_out may replace the residual in place
    assert lib.tw_add_rmsnorm(A, A + 10 * MB, A + 11 * MB, A + 12 * MB, A + 10 * MB, 4, 64,
                              ctypes.c_float(-1.0), 1, None) == INVALID
    assert b"eps" in lib.tw_last_error()
    assert lib.tw_add_rmsnorm(0, 0, 0, 0, 0, 0, 64, ctypes.c_float(1e-5), 1, None) == 0


def test_grid_entry_validates_workgroups(lib):
    parts = (ctypes.c_void_p * 2)(A, A + MB)
    args = [parts, 2, A + 10 * MB, A + 11 * MB, A + 12 * MB, A + 13 * MB, 4, 64,
            ctypes.c_float(1e-5), 1]
    for g in (0, -3):
        assert lib.tw_fused_reduce_rmsnorm_grid(*args, g, None) == INVALID
        assert b"num_workgroups" in lib.tw_last_error()
    bad = list(args)
    bad[8] = ctypes.c_float(-1.0)
    assert lib.tw_fused_reduce_rmsnorm_grid(*bad, 8, None) == INVALID


def test_pointer_checks_reject_unknown_memory(lib):
    # With checks on, pointers the HIP runtime does not know (here: fake
    # addresses, with no GPU at all) are rejected before any launch.
    tw.tw_set_pointer_checks(True)
    try:
        assert _call(lib) == INVALID
        assert b"partials[0]" in lib.tw_last_error()
        assert _call(lib, T=0) == 0            # nothing to launch, nothing checked
    finally:
        tw.tw_set_pointer_checks(False)
    assert _call(lib, eps=-1.0) == INVALID     # plain validation still first
    assert b"eps" in lib.tw_last_error()


def test_shard_index_range(lib):
    for k in (-1, 2, 100):
        assert _call(lib, shard=k) == INVALID
        assert b"shard_index" in lib.tw_last_error()


def test_empty_batch_is_a_noop(lib):
    # T == 0 returns OK without looking at the pointers (and without a launch).
    assert _call(lib, T=0, parts=[0, 0], res=0, w=0, out=0, rout=0) == 0
    assert _call(lib, T=0, parts=[0, 0], res=0, w=0, out=0, rout=0, shard=1) == 0


def test_adjacent_buffers_do_not_overlap(lib):
    # T*h*2 = 512 bytes: a tensor ending where the next begins is not an overlap;
    # still invalid elsewhere (eps) so nothing launches.
    T, h = 4, 64
    nb = T * h * 2
    r = _call(lib, T=T, h=h, parts=[A, A + nb], res=A + 2 * nb, w=A + 3 * nb,
              out=A + 3 * nb + h * 2, rout=A + 4 * nb + h * 2, eps=-1.0)
    assert r == INVALID and b"eps" in lib.tw_last_error()


def test_in_place_residual_is_allowed_by_validation(lib):
    # residual_out == residual passes the overlap check (with pointer checks
    # on, the fake addresses are then rejected as unknown memory, not as an
    # overlap); out == residual and a shifted residual_out are not allowed.
    tw.tw_set_pointer_checks(True)
    try:
        assert _call(lib, rout=A + 10 * MB) == INVALID
        assert b"overlap" not in lib.tw_last_error()
    finally:
        tw.tw_set_pointer_checks(False)
    assert _call(lib, out=A + 10 * MB) == INVALID
    assert b"out overlaps residual" in lib.tw_last_error()
    assert _call(lib, rout=A + 10 * MB + 16) == INVALID
    assert b"residual_out overlaps residual" in lib.tw_last_error()


# --------------------------------------------------------------- planner ----

def _both(T, **kw):
    return tw.tw_split_plan(T, **kw), oracle.split_plan(T, **kw)


def test_planner_matches_oracle_exhaustive():
    for S in (132, 256, 7, 1):
        for T in range(0, 601):
            got, want = _both(T, num_cus=S)
            assert got == want, (S, T)


def test_planner_matches_oracle_random_tile_models():
    rng = random.Random(11)
    for _ in range(3000):
        kw = dict(tokens_per_cta=rng.choice([1, 16, 64, 128, 256]),
                  ctas_per_token_tile=rng.choice([1, 2, 8, 32, 64]),
                  num_cus=rng.choice([1, 8, 132, 256, 304]),
                  ctas_per_cu=rng.choice([1, 2, 4]),
                  min_split_tokens=rng.choice([0, 1024, 4096]))
        if rng.random() < 0.3:
            kw["offsets"] = sorted(rng.sample(range(0, 1500), rng.randint(0, 8)))
        T = rng.choice([rng.randint(0, 70000), rng.randint(0, 5000), 2 ** rng.randint(0, 16)])
        got, want = _both(T, **kw)
        assert got == want, (T, kw)


def test_planner_workload_tile_model():
    # GEMM tile model used for the Qwen2.5-72B-shaped split: 256x256 tiles over
    # 8192 output features (32 tiles), one CTA per CU, 256 CUs.
    p = tw.tw_split_plan(4096, tokens_per_cta=256, ctas_per_token_tile=32, num_cus=256,
                         min_split_tokens=1024)
    assert (p["prefix_tokens"], p["suffix_tokens"], p["offset"], p["reason"]) == (2048, 2048, 0, 0)
    p = tw.tw_split_plan(1024, tokens_per_cta=256, ctas_per_token_tile=32, num_cus=256,
                         min_split_tokens=1024)
    assert p["reason"] == 2


@pytest.mark.parametrize("kw", [
    dict(num_tokens=-1), dict(tokens_per_cta=0), dict(ctas_per_token_tile=0), dict(num_cus=0),
    dict(ctas_per_cu=0), dict(min_split_tokens=-5), dict(offsets=[0, 64, 64]),
    dict(offsets=[64, 0]), dict(offsets=[-64, 0]),
])
def test_planner_invalid(kw):
    args = dict(num_tokens=100)
    args.update(kw)
    T = args.pop("num_tokens")
    with pytest.raises(tw.TokenWeaveError) as e:
        tw.tw_split_plan(T, **args)
    assert e.value.status == INVALID


def test_planner_null_and_limits(lib):
    res = _lib.SplitPlanResult()
    assert lib.tw_split_plan(None, ctypes.byref(res)) == INVALID
    prob = _lib.SplitProblem(10, 1, 1, 256, 1, 0, None, 3)      # NULL offsets with a length
    assert lib.tw_split_plan(ctypes.byref(prob), ctypes.byref(res)) == INVALID
    assert lib.tw_split_plan(ctypes.byref(prob), None) == INVALID
    with pytest.raises(tw.TokenWeaveError) as e:
        tw.tw_split_plan(2 ** 41)
    assert e.value.status == UNSUPPORTED
    with pytest.raises(tw.TokenWeaveError) as e:
        tw.tw_split_plan(10, ctas_per_token_tile=2 ** 21)
    assert e.value.status == UNSUPPORTED
    with pytest.raises(tw.TokenWeaveError) as e:    # 2^40 waves do not fit int32
        tw.tw_split_plan(2 ** 40, num_cus=1)
    assert e.value.status == UNSUPPORTED


def test_overlap_validation_matches_brute_force(lib):
    # Random placements of 2 partials, residual, weight, out and residual_out
    # on a small grid of 16-byte-aligned addresses.  With pointer checks on, a
    # layout that passes the overlap rule stops at "memory the runtime does
    # not know" (fake addresses), so nothing ever launches; a layout that
    # breaks it must be reported as an overlap.  The rule: an output may not
    # share a byte with any other tensor, except residual_out == residual.
    rng = random.Random(5)
    T, h = 2, 64
    tb, wb = T * h * 2, h * 2
    tw.tw_set_pointer_checks(True)
    try:
        for _ in range(600):
            addr = {k: A + 16 * rng.randrange(0, 96) for k in ("p0", "p1", "res", "w", "out", "rout")}
            if rng.random() < 0.2:
                addr["rout"] = addr["res"]
            size = {"p0": tb, "p1": tb, "res": tb, "w": wb, "out": tb, "rout": tb}

            def ov(a, b):
                return addr[a] < addr[b] + size[b] and addr[b] < addr[a] + size[a]
            bad = False
            for o in ("out", "rout"):
                for k in size:
                    if k == o or (o == "rout" and k == "res" and addr["rout"] == addr["res"]):
                        continue
                    bad |= ov(o, k)
            st = _call(lib, T=T, h=h, parts=[addr["p0"], addr["p1"]], res=addr["res"], w=addr["w"],
                       out=addr["out"], rout=addr["rout"])
            msg = lib.tw_last_error().decode()
            assert st == INVALID, (addr, st, msg)
            assert ("overlaps" in msg) == bad, (addr, msg)
    finally:
        tw.tw_set_pointer_checks(False)


def test_last_error_is_per_thread(lib):
    # Each host thread sees the message of its own last failing call.
    import threading
    results = {}

    def worker(k):
        for _ in range(200):
            if k == 0:
                _call(lib, eps=-1.0)
            else:
                _call(lib, h=12)
            results.setdefault(k, set()).add(lib.tw_last_error())

    threads = [threading.Thread(target=worker, args=(k,)) for k in (0, 1)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert all(b"eps" in m for m in results[0])
    assert all(b"multiple" in m for m in results[1])


def test_plan_constants_match_the_header():
    text = open(os.path.join(os.path.dirname(_lib.LIB_PATH), "..", "include", "tokenweave.h")).read()
    names = ("TW_PLAN_SPLIT", "TW_PLAN_BELOW_THRESHOLD", "TW_PLAN_SINGLE_WAVE",
             "TW_PLAN_NO_FEASIBLE_OFFSET", "TW_PLAN_EMPTY", "TW_PLAN_MEASURED_SPLIT",
             "TW_PLAN_MEASURED_UNSPLIT", "TW_PLAN_MEASURED_OVER_WAVES")
    for name in names:
        m = re.search(rf"#define {name} (\d+)", text)
        assert m and int(m.group(1)) == getattr(_lib, name), name
        assert tw.PLAN_REASONS[getattr(_lib, name)]
        assert getattr(oracle, "REASON" + name[len("TW_PLAN"):]) == getattr(_lib, name)
    assert len({getattr(_lib, n) for n in names}) == len(names)


# The offline sweep's table (fastest offset per token count, -1 for the whole
# batch) of one Llama-3-70B-shaped layer step: 256 x 256 GEMM tiles, 32 across
# h = 8192, 256 CUs, threshold 1024.  It lists a count whose measured offset
# breaks the wave bound (5632 at offset 128: 2 + 2 waves against 3).
MEASURED_SWEEP = {1024: -1, 1536: -1, 2048: -1, 2560: -1, 3072: -1, 3584: -1, 4096: -1,
                  4608: -1, 5120: 512, 5632: 128, 6144: -1, 6656: 192, 7168: 256, 7680: 256,
                  8192: -1}
SWEEP_MODEL = dict(tokens_per_cta=256, ctas_per_token_tile=32, num_cus=256, ctas_per_cu=1,
                   min_split_tokens=1024)


def test_measured_plan_matches_the_oracle_on_the_sweep_table():
    # Every listed count and every count between them, bit-exact in every field.
    for T in sorted(set(MEASURED_SWEEP) | set(range(0, 8400, 64))):
        assert tw.tw_split_plan_measured(T, MEASURED_SWEEP, **SWEEP_MODEL) == \
            oracle.split_plan_measured(T, MEASURED_SWEEP, **SWEEP_MODEL), T
    p = tw.tw_split_plan_measured(5632, MEASURED_SWEEP, **SWEEP_MODEL)
    assert p["reason"] == _lib.TW_PLAN_MEASURED_OVER_WAVES and p["suffix_tokens"] == 0
    p = tw.tw_split_plan_measured(5120, MEASURED_SWEEP, **SWEEP_MODEL)
    assert (p["prefix_tokens"], p["suffix_tokens"], p["reason"]) == \
        (3072, 2048, _lib.TW_PLAN_MEASURED_SPLIT)


def test_measured_plan_matches_the_oracle_on_random_tables():
    rng = random.Random(11)
    for _ in range(300):
        cus = rng.choice([7, 64, 132, 256])
        kw = dict(tokens_per_cta=rng.choice([1, 16, 128]), ctas_per_token_tile=rng.choice([1, 3, 32]),
                  num_cus=cus, ctas_per_cu=rng.choice([1, 2]),
                  min_split_tokens=rng.choice([0, 100, 1024]))
        counts = sorted(rng.sample(range(1, 5000), rng.randint(0, 12)))
        table = {t: rng.choice([-1] + [o for o in (0, 1, 64, 100, 300, 999) if o < t // 2])
                 for t in counts}
        arr = tw.split_table(table)
        for T in counts + [rng.randint(0, 5000) for _ in range(5)]:
            assert tw.tw_split_plan_measured(T, arr, **kw) == \
                oracle.split_plan_measured(T, table, **kw), (T, table, kw)


def test_measured_plan_with_an_empty_table_is_the_analytic_plan():
    for T in range(0, 700, 7):
        assert tw.tw_split_plan_measured(T, {}, num_cus=132) == tw.tw_split_plan(T, num_cus=132)


def test_measured_plan_rejects_bad_tables(lib):
    for bad in ({100: 50}, {100: -2}, {0: -1}, {101: 50}):
        with pytest.raises(tw.TokenWeaveError) as e:
            tw.tw_split_plan_measured(100, bad)
        assert e.value.status == INVALID
    # not ascending, duplicated, negative length, NULL with a length
    unsorted = (_lib.SplitEntry * 2)(_lib.SplitEntry(200, 0), _lib.SplitEntry(100, 0))
    dup = (_lib.SplitEntry * 2)(_lib.SplitEntry(100, 0), _lib.SplitEntry(100, 1))
    prob, _ = _lib._split_problem(100, 1, 1, 256, 1, 0, None)
    res = _lib.SplitPlanResult()
    for arr, n in ((unsorted, 2), (dup, 2), (dup, -1), (None, 3)):
        assert lib.tw_split_plan_measured(ctypes.byref(prob), arr, n, ctypes.byref(res)) == INVALID
    assert lib.tw_split_plan_measured(None, dup, 1, ctypes.byref(res)) == INVALID
    assert lib.tw_split_plan_measured(ctypes.byref(prob), dup, 1, None) == INVALID


def test_split_plan_cache_with_a_measured_table():
    # The cache only stores the C planner's plans: the table's split where it
    # meets the wave bound, the whole batch where the table says so or where
    # its offset breaks the bound, and the analytic plan elsewhere.
    cache = tw.SplitPlanCache(measured=MEASURED_SWEEP, **SWEEP_MODEL)
    for T in (1024, 3072, 5120, 5632, 6656, 6000, 8192, 9000):
        assert cache(T) == oracle.split_plan_measured(T, MEASURED_SWEEP, **SWEEP_MODEL)
    got = cache(5120)
    got["prefix_tokens"] = 0                                           # a copy: the table keeps its plan
    assert cache(5120)["prefix_tokens"] == 3072
    table = tw.split_table_from_sweep([{"tokens": 5632, "fastest": 128},
                                       {"tokens": 4096, "fastest": -1}])
    assert table == {5632: 128, 4096: -1}
    for bad in ({100: 50}, {100: -2}, {0: -1}):
        with pytest.raises(tw.TokenWeaveError):
            tw.SplitPlanCache(measured=bad, **SWEEP_MODEL)
