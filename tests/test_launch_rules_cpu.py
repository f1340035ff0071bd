"""The fused launcher's choice of kernel per dispatch (one workgroup per row
with all loads at once, one workgroup per row loading the tensors in
sequence, or the strided kernel), checked at the shapes where the choice was
measured on MI355X.  tests/c/launch_rules.cpp is built with the host
compiler against the launcher's geometry header; no GPU.

A round is the number of workgroups resident at once on the CUs a launch
may use; on 256 CUs: 512 for the 1024-thread geometries, 1024 for 512 x 1
and 512 x 3, 768 for 640 x 1, 1280 for 384 x 1 and 1536 for 320 x 1.  The
rules:
* below one round, all loads at once (too few rows to fill the CUs);
* between one and one and a half rounds, all loads at once when each thread
  waits on a chain of 8 or more tensors (N + 1 tensors, one or two in
  flight), since the rows past the first round run almost alone;
* from one to four rounds with a last round at most half full, the strided
  kernel (one round of workgroups, each taking every round-th row), where the
  geometry loads all of a thread's vector slots in one sequence;
* otherwise the sequenced one-row kernel.
Geometries without a sequenced order always load everything at once.  The
1024 x 2 geometry (h = 16384 bf16, and 9216-12288 below six partials) loads
both of a thread's vector slots at once, rather than one after the other,
when a launch gives more than seven eighths of the CUs one workgroup each and
none two, with up to 11 partials ("both")."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "launch_rules.cpp")
CSRC = os.path.join(ROOT, "reduce_rmsnorm_amd", "csrc")

# (hidden, element bytes, N, rows) -> kernel
CASES = {
    # h = 8192 bf16: 1024 x 1 from N = 5 on (two tensors in flight for N = 5, 6)
    (8192, 2, 8, 128): "all", (8192, 2, 8, 511): "all", (8192, 2, 8, 512): "seq",
    (8192, 2, 8, 513): "all", (8192, 2, 8, 520): "all", (8192, 2, 8, 576): "all",
    (8192, 2, 8, 640): "all", (8192, 2, 8, 700): "all", (8192, 2, 8, 767): "all",
    (8192, 2, 8, 768): "strided", (8192, 2, 8, 769): "seq", (8192, 2, 8, 896): "seq",
    (8192, 2, 8, 1024): "seq", (8192, 2, 8, 1025): "strided", (8192, 2, 8, 1100): "strided",
    (8192, 2, 8, 1280): "strided", (8192, 2, 8, 1281): "seq", (8192, 2, 8, 1536): "seq",
    (8192, 2, 8, 1792): "strided", (8192, 2, 8, 2047): "seq", (8192, 2, 8, 2048): "seq",
    (8192, 2, 8, 2100): "seq", (8192, 2, 8, 4096): "seq",
    (8192, 2, 7, 600): "all", (8192, 2, 16, 700): "all", (8192, 2, 12, 600): "all",
    (8192, 2, 5, 600): "strided", (8192, 2, 6, 600): "strided", (8192, 2, 6, 1024): "seq",
    (8192, 2, 4, 1024): "all", (8192, 2, 2, 4096): "all", (8184, 2, 7, 700): "all",
    (8184, 2, 7, 1200): "strided",
    # h = 4096 bf16: 512 x 1, one tensor in flight from N = 2 on
    (4096, 2, 8, 1023): "all", (4096, 2, 8, 1024): "seq", (4096, 2, 8, 1040): "all",
    (4096, 2, 8, 1400): "all", (4096, 2, 8, 1535): "all", (4096, 2, 8, 1536): "strided",
    (4096, 2, 8, 1600): "seq", (4096, 2, 8, 2560): "strided", (4096, 2, 8, 8192): "seq",
    (4096, 2, 2, 1100): "strided", (4096, 2, 2, 1300): "strided", (4096, 2, 1, 4096): "all",
    (4096, 2, 6, 1100): "strided", (4096, 2, 7, 1100): "all", (4096, 2, 3, 1100): "strided",
    # h = 16384 bf16: 1024 x 2, one vector slot at a time, no strided kernel
    (16384, 2, 8, 256): "both", (16384, 2, 8, 224): "all", (16384, 2, 8, 225): "both",
    (16384, 2, 8, 257): "all", (16384, 2, 11, 256): "both", (16384, 2, 12, 256): "all",
    (16384, 2, 4, 240): "both", (12288, 2, 4, 256): "both", (12288, 2, 8, 256): "all",
    (16384, 2, 8, 128): "all", (16384, 2, 8, 512): "seq", (16384, 2, 8, 576): "all",
    (16384, 2, 8, 640): "all", (16384, 2, 8, 768): "seq", (16384, 2, 8, 1100): "seq",
    (16384, 2, 1, 2048): "all",
    # float32: h = 4096 is the 1024 x 1 class, h = 8192 the 1024 x 2 class
    (4096, 4, 8, 640): "all", (4096, 4, 8, 1100): "strided", (4096, 4, 12, 1700): "strided",
    (8192, 4, 7, 600): "all", (8192, 4, 2, 600): "seq",
    # widths between the powers of two: 320, 384 and 640 threads, one vector
    # each (640 only from N = 7 on; below, the 512 x 2 class's geometry)
    (2560, 2, 8, 1536): "seq", (2560, 2, 8, 1600): "all", (2560, 2, 2, 1600): "strided",
    (2560, 2, 8, 1535): "all", (3072, 2, 2, 1280): "seq", (3072, 2, 8, 1400): "all",
    (5120, 2, 8, 768): "seq", (5120, 2, 8, 800): "all", (5120, 2, 8, 1600): "strided",
    (5120, 2, 7, 1100): "all", (5120, 2, 6, 1100): "strided", (5120, 2, 4, 1100): "all",
    (1280, 4, 4, 3100): "strided", (1280, 4, 8, 1600): "all",
    # 1025-1536 vectors: 512 x 3 from N = 6 on (no strided kernel: one slot at
    # a time), 1024 x 2 below
    (12288, 2, 8, 1024): "seq", (12288, 2, 8, 1100): "all", (12288, 2, 8, 2200): "seq",
    (12288, 2, 8, 256): "all", (12288, 2, 4, 1100): "seq", (9216, 2, 16, 1600): "seq",
    # narrow and wide rows never load in sequence
    (512, 4, 2, 64): "all", (2048, 2, 8, 100000): "all", (32768, 2, 8, 4096): "all",
}


@pytest.fixture(scope="module")
def rules_exe(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("rules") / "launch_rules")
    subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-Wextra", "-Werror", "-I", CSRC, SRC,
                    "-o", exe], check=True, capture_output=True, text=True)
    return exe


def _run(exe, cases, cus=256):
    stdin = "".join(f"{h} {es} {n} {rows} {cus}\n" for h, es, n, rows in cases)
    out = subprocess.run([exe], input=stdin, check=True, capture_output=True, text=True).stdout
    return [line.split() for line in out.splitlines()]


def test_kernel_choice_at_the_measured_shapes(rules_exe):
    keys = list(CASES)
    got = _run(rules_exe, keys)
    assert len(got) == len(keys)
    bad = [(k, CASES[k], g[0]) for k, g in zip(keys, got) if g[0] != CASES[k]]
    assert not bad, bad


def test_round_sizes(rules_exe):
    # (threads, vectors per thread) and the rows one round holds
    got = _run(rules_exe, [(8192, 2, 8, 1), (4096, 2, 8, 1), (16384, 2, 8, 1), (8192, 2, 4, 1),
                           (2560, 2, 8, 1), (3072, 2, 8, 1), (5120, 2, 8, 1), (5120, 2, 6, 1),
                           (5120, 2, 4, 1), (5112, 2, 16, 1), (2552, 2, 1, 1),
                           (12288, 2, 8, 1), (12288, 2, 4, 1), (12288, 2, 1, 1)])
    assert [g[1:] for g in got] == [["1024", "1", "512"], ["512", "1", "1024"],
                                    ["1024", "2", "512"], ["512", "2", "1024"],
                                    ["320", "1", "1536"], ["384", "1", "1280"],
                                    ["640", "1", "768"], ["1024", "1", "512"],
                                    ["512", "2", "1024"], ["640", "1", "768"],
                                    ["320", "1", "1536"], ["512", "3", "1024"],
                                    ["1024", "2", "512"], ["512", "4", "1024"]]


def test_strided_kernel_only_within_four_rounds_with_a_short_last_round(rules_exe):
    # Every row count from 1 to 5 rounds: the strided kernel exactly where
    # its rule holds, and all loads at once only below 1.5 rounds.
    cases = [(8192, 2, 8, r) for r in range(1, 5 * 512 + 1)]
    for (h, es, n, rows), g in zip(cases, _run(rules_exe, cases)):
        tail = rows % 512
        strided = 512 < rows < 2048 and 0 < tail <= 256 and 2 * rows >= 3 * 512
        everything = rows < 512 or 512 < rows < 768
        want = "strided" if strided else "all" if everything else "seq"
        assert g[0] == want, (rows, g[0], want)


@pytest.mark.parametrize("cus", [8, 32, 64, 128, 192, 255, 256, 304])
def test_rules_scale_with_the_cu_count(rules_exe, cus):
    # The same rules on any CU count: the round is cus x (2048 / threads), so
    # a 1024-thread class holds 2 rows per CU, and every row count from 1 to
    # 5 rounds takes the kernel the rules give for that round.
    rnd = 2 * cus
    cases = [(8192, 2, 8, r) for r in range(1, 5 * rnd + 1)]
    for (h, es, n, rows), g in zip(cases, _run(rules_exe, cases, cus)):
        assert g[1:] == ["1024", "1", str(rnd)]
        tail = rows % rnd
        strided = rnd < rows < 4 * rnd and 0 < tail and 2 * tail <= rnd and 2 * rows >= 3 * rnd
        everything = rows < rnd or rnd < rows and 2 * rows < 3 * rnd
        want = "strided" if strided else "all" if everything else "seq"
        assert g[0] == want, (cus, rows, g[0], want)


def test_measured_shapes_scale_with_the_cu_count(rules_exe):
    # Scaling a 256-CU case's rows by cus / 256 (whole rounds stay whole)
    # gives the same kernel on cus CUs.
    keys = [k for k in CASES if k[3] % 4 == 0]
    for cus in (64, 128):
        scaled = [(h, es, n, rows * cus // 256) for h, es, n, rows in keys]
        got = _run(rules_exe, scaled, cus)
        bad = [(k, CASES[k], g[0]) for k, g in zip(keys, got) if g[0] != CASES[k]]
        assert not bad, (cus, bad)


def test_library_launch_info_matches_the_rules(rules_exe):
    # The library's own view of a launch (tw_fused_launch_info) takes the
    # same rules: checked against the rule program at the measured shapes, on
    # the CU count the library counts for the null stream (every CU of the
    # device; 256 where the runtime cannot say, as without a GPU).
    import torch
    import reduce_rmsnorm_amd as tw
    first = tw.tw_fused_launch_info(8, 1024, 8192)
    cus = first["num_cus"]
    keys = list(CASES)
    got = _run(rules_exe, keys, cus)
    for (h, es, n, rows), g in zip(keys, got):
        info = tw.tw_fused_launch_info(n, rows, h, torch.bfloat16 if es == 2 else torch.float32)
        assert info["num_cus"] == cus
        assert (info["threads_per_workgroup"], info["vectors_per_thread"], info["round_rows"]) == \
            (int(g[1]), int(g[2]), int(g[3]))
        if info["dispatches"] == 1:
            assert info["kernel_name"] == g[0], (h, es, n, rows)
    if cus == 256:
        assert [(k, tw.tw_fused_launch_info(k[2], k[3], k[0])["kernel_name"]) for k in
                [(8192, 2, 8, 1024), (8192, 2, 8, 700), (8192, 2, 8, 1280)]] == \
            [((8192, 2, 8, 1024), "seq"), ((8192, 2, 8, 700), "all"), ((8192, 2, 8, 1280), "strided")]


def test_library_launch_info_cuts_long_calls():
    import reduce_rmsnorm_amd as tw
    info = tw.tw_fused_launch_info(8, 70_000_000, 8)          # 16-byte rows, N = 8
    assert info["dispatches"] > 1
    assert info["rows_per_dispatch"] * info["dispatches"] >= 70_000_000
    assert info["rows_per_dispatch"] * info["threads_per_workgroup"] <= 2 ** 31 - 1
    none = tw.tw_fused_launch_info(8, 0, 8192)
    assert (none["dispatches"], none["rows_per_dispatch"], none["kernel"]) == (0, 0, -1)
    with pytest.raises(tw.TokenWeaveError):
        tw.tw_fused_launch_info(0, 10, 8192)
    with pytest.raises(tw.TokenWeaveError):
        tw.tw_fused_launch_info(8, 10, 12)
