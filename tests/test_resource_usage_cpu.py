"""Register and scratch use of the built kernels, from the compiler's
resource report that the build keeps (``_build/*.resources.txt``).  No GPU.

Scratch here means registers spilled to memory, which a memory-bound kernel
pays for in traffic.  No fused kernel of rows up to 4096 vectors (h = 32768
bf16) may spill, in any load order or partial count; the consecutive-rows
kernel of the grid entry may not spill at the widths its footprint
measurements use (up to 1024 vectors, h = 8192 bf16).  The widest class (1024
x 8, rows of 4097-8192 vectors) and the grid kernel's wide classes hold a
whole row in registers and do spill; their known extents are listed, so that
a new spill anywhere fails."""

import os
import re

import pytest

from reduce_rmsnorm_amd import build as B

ONE_ROW = re.compile(r"fused_reduce_rmsnorm_(kernel|strided_kernel)ILi(\d+)ELi(\d+)ELi(\d+)ELb([01])"
                     r"ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E")
ROWS = re.compile(r"fused_reduce_rmsnorm_rows_kernelILi(\d+)ELi(\d+)ELi(\d+)ELb([01])ELi(\d+)"
                  r"ELi(\d+)ELi(\d+)E")
# (kernel, threads, vectors per thread, bf16) -> the partial counts that spill
KNOWN_SPILLS = {
    ("one-row", 1024, 8, 1): set(range(1, 17)),
    ("rows", 1024, 8, 0): set(range(1, 17)),
    ("rows", 1024, 8, 1): set(range(1, 17)),
    ("rows", 1024, 4, 0): set(range(6, 17)),
    ("rows", 1024, 4, 1): set(range(4, 17)),
    ("rows", 1024, 2, 0): set(range(13, 17)),
    ("rows", 1024, 2, 1): set(range(11, 17)),
}


def _report(src):
    path = B.resource_report(src)
    if not os.path.exists(path):
        pytest.skip(f"{path} missing: build the library first")
    blocks = re.split(r"\n(?=.*Function Name:)", open(path).read())
    out = []
    for b in blocks:
        m = re.search(r"Function Name: (\S+)", b)
        if not m:
            continue
        scratch = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", b)
        vgpr = re.search(r"VGPRs: (\d+)", b)
        occ = re.search(r"Occupancy \[waves/SIMD\]: (\d+)", b)
        out.append((m.group(1), int(scratch.group(1)), int(vgpr.group(1)), int(occ.group(1))))
    return out


def test_fused_kernels_spill_only_where_listed():
    seen = 0
    spills = {}
    for name, scratch, _, _ in _report("fused_reduce_rmsnorm.hip"):
        m, r = ONE_ROW.search(name), ROWS.search(name)
        if m:
            kind, n, block, vpt, bf16 = "one-row", int(m[2]), int(m[3]), int(m[4]), int(m[5])
        elif r:
            kind, n, block, vpt, bf16 = "rows", int(r[1]), int(r[2]), int(r[3]), int(r[4])
        else:
            continue
        seen += 1
        if scratch:
            spills.setdefault((kind, block, vpt, bf16), set()).add(n)
    assert seen > 500
    for key, ns in spills.items():
        assert ns <= KNOWN_SPILLS.get(key, set()), (key, sorted(ns))


def test_workload_kernels_use_no_scratch_at_full_occupancy():
    # The kernels the benchmark's workloads run, in every load order their
    # launches take: N = 8 bf16 at h = 8192 (1024 x 1), 4096 (512 x 1) and
    # 16384 (1024 x 2), and N = 2 float32 at h = 512 (128 x 1).
    want = {(8, 1024, 1, 1), (8, 512, 1, 1), (8, 1024, 2, 1), (2, 128, 1, 0)}
    found = set()
    for name, scratch, vgpr, occ in _report("fused_reduce_rmsnorm.hip"):
        m = ONE_ROW.search(name)
        if not m:
            continue
        key = (int(m[2]), int(m[3]), int(m[4]), int(m[5]))
        if key in want:
            found.add(key)
            assert scratch == 0, name
            if key[1] * key[2] > 128 and int(m[6]) == 8:
                assert occ >= 8, (name, occ)
    assert found == want


def test_comparator_kernels_use_no_scratch():
    rows = _report("unfused.hip")
    assert rows
    for name, scratch, _, _ in rows:
        if re.search(r"ILi(\d+)ELi1024ELi8E", name):
            continue                                    # the 1024 x 8 class holds a whole row
        assert scratch == 0, name
