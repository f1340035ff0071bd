"""The C ABI from plain C: tests/c/abi_check.c is compiled as C99 (and, to
check the header's C++ guards, as C++11) against include/tokenweave.h and
linked with the built library.  Its planner results (analytic, and with a
measured table) must match the oracle field for field, and its argument checks must return the documented status
codes.  No device work: runs without a GPU."""

import os
import random
import shutil
import subprocess

import pytest

import oracle
from reduce_rmsnorm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "abi_check.c")
FIELDS = ("prefix_tokens", "suffix_tokens", "offset", "waves_unsplit", "waves_prefix",
          "waves_suffix", "reason")

# status codes the header documents for each case abi_check.c runs
EXPECTED_STATUS = {
    "null_partials": _lib.TW_ERR_INVALID_ARG,
    "hidden_not_16_bytes": _lib.TW_ERR_UNSUPPORTED,
    "negative_eps": _lib.TW_ERR_INVALID_ARG,
    "shard_index_out_of_range": _lib.TW_ERR_INVALID_ARG,
    "out_overlaps_partial": _lib.TW_ERR_INVALID_ARG,
    "empty_batch": _lib.TW_OK,
    "plan_null_problem": _lib.TW_ERR_INVALID_ARG,
    "plan_zero_tile": _lib.TW_ERR_INVALID_ARG,
    "plan_table_not_ascending": _lib.TW_ERR_INVALID_ARG,
    "plan_table_offset_at_half": _lib.TW_ERR_INVALID_ARG,
    "plan_table_null": _lib.TW_ERR_INVALID_ARG,
    "randomized_refused": 0,      # 0: every randomized invalid call was refused
}


def _build(tmp_path, compiler, std, lang):
    exe = str(tmp_path / f"abi_check_{lang}")
    libdir = os.path.dirname(_lib.LIB_PATH)
    cmd = [compiler, f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic", "-x", lang, SRC,
           "-x", "none", "-I", os.path.join(ROOT, "include"), "-L", libdir, "-ltokenweave",
           f"-Wl,-rpath,{libdir}", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


@pytest.fixture(scope="module")
def cases():
    rnd = random.Random(5)
    c = [(257, 1, 1, 256, 1, 0), (514, 1, 1, 256, 1, 0), (300, 1, 1, 132, 1, 0),
         (393, 1, 1, 132, 1, 0), (0, 1, 1, 256, 1, 0), (100, 1, 1, 256, 1, 1024),
         (4096, 256, 32, 256, 1, 1024), (8192, 256, 16, 256, 1, 4096),
         # extreme tile models: no wave arithmetic may overflow int64 on the way
         (2 ** 40, 2 ** 63 - 1, 1, 256, 1, 0), (5000, 2 ** 63 - 1, 2 ** 20, 1, 1, 0),
         (2 ** 40, 1, 1, 2 ** 31 - 1, 2 ** 31 - 1, 0), (2 ** 40, 2 ** 62, 2 ** 20, 2 ** 31 - 1, 1, 0),
         (70000, 2 ** 63 - 1, 64, 256, 4, 1024)]
    for _ in range(300):
        c.append((rnd.randint(0, 70000), rnd.choice([1, 64, 128, 256]), rnd.randint(1, 64),
                  rnd.choice([132, 256, 304]), rnd.randint(1, 4), rnd.choice([0, 1024, 4096])))
    # each case also carries a one-entry measured table: its own token count
    # (with an offset that may or may not meet the wave bound), or another one
    out = []
    for k, case in enumerate(c):
        T = case[0]
        if T >= 2 and k % 3 != 2:
            off = rnd.choice([-1] + [o for o in (0, 64, 128, 512, T // 2 - 1)
                                     if 0 <= o < min(T // 2, 2 ** 31)])
            out.append(case + (T, off))
        else:
            out.append(case + (T + 1000, -1))
    return out


def _want(case):
    T, tpc, tiles, cus, occ, thr, tab_t, tab_off = case
    kw = dict(tokens_per_cta=tpc, ctas_per_token_tile=tiles, num_cus=cus, ctas_per_cu=occ,
              min_split_tokens=thr)
    return ([_lib.TW_OK] + [oracle.split_plan(T, **kw)[f] for f in FIELDS] + [_lib.TW_OK] +
            [oracle.split_plan_measured(T, {tab_t: tab_off}, **kw)[f] for f in FIELDS])


@pytest.mark.parametrize("compiler,std,lang", [("gcc", "c99", "c"), ("g++", "c++11", "c++")])
def test_c_program_matches_oracle(tmp_path, cases, compiler, std, lang):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not installed")
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail(f"{_lib.LIB_PATH} is missing: build it first")
    exe = _build(tmp_path, compiler, std, lang)
    stdin = "".join(" ".join(str(v) for v in c) + "\n" for c in cases)
    run = subprocess.run([exe], input=stdin, capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    lines = run.stdout.splitlines()
    assert lines[-1] == "done"
    for c, ln in zip(cases, lines[:len(cases)]):
        assert [int(v) for v in ln.split()] == _want(c), (c, ln)
    checks = dict(ln.split() for ln in lines[len(cases):-1])
    assert {k: int(v) for k, v in checks.items()} == EXPECTED_STATUS


def test_c_program_under_address_and_undefined_sanitizers(tmp_path, cases):
    """The host code (argument validation, split planner) built with
    AddressSanitizer and UndefinedBehaviorSanitizer, driven by the same C
    program: every planner case, every error path and 2000 randomized invalid
    calls, with no sanitizer report.  Host code only: the kernels are linked
    from the regular build and never launched."""
    from reduce_rmsnorm_amd import build as B
    objs = [os.path.join(B.BUILD, s + ".o") for s in B.HIP_SOURCES]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects not built (run the build first)")
    for tool in ("gcc", "g++"):
        if shutil.which(tool) is None:
            pytest.skip(f"{tool} not installed")
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
    host = []
    for src in B.HOST_SOURCES:
        o = str(tmp_path / (src + ".o"))
        subprocess.run(["g++", "-std=c++17", *san, "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        "-I", os.path.join(ROOT, "include"), "-c", os.path.join(B.CSRC, src), "-o", o],
                       check=True, capture_output=True, text=True)
        host.append(o)
    main_o = str(tmp_path / "abi_check.o")
    subprocess.run(["gcc", "-std=c99", *san, "-I", os.path.join(ROOT, "include"), "-c", SRC, "-o", main_o],
                   check=True, capture_output=True, text=True)
    exe = str(tmp_path / "abi_check_san")
    link = subprocess.run(["g++", *san, main_o, *host, *objs, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib",
                           "-lamdhip64", "-o", exe], capture_output=True, text=True)
    if link.returncode != 0:
        pytest.skip(f"sanitizer link unavailable: {link.stderr[-300:]}")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    stdin = "".join(" ".join(str(v) for v in c) + "\n" for c in cases)
    run = subprocess.run([exe], input=stdin, capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0, run.stderr[-2000:]
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-2000:]
    lines = run.stdout.splitlines()
    assert lines[-1] == "done"
    for c, ln in zip(cases, lines[:len(cases)]):
        assert [int(v) for v in ln.split()] == _want(c), (c, ln)
    checks = dict(ln.split() for ln in lines[len(cases):-1])
    assert {k: int(v) for k, v in checks.items()} == EXPECTED_STATUS
