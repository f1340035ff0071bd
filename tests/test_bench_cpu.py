"""bench.py's contract checks that need no GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert run.returncode == 2
    assert "one GPU" in run.stderr + run.stdout
    assert run.stdout.strip() == ""          # no JSON line


def test_kernel_code_hash_ignores_comments_and_catches_code(tmp_path):
    sys.path.insert(0, ROOT)
    from reduce_rmsnorm_amd.rocprof_summary import KERNEL_SOURCES, kernel_code_hash
    copies = []
    for p in KERNEL_SOURCES:
        q = tmp_path / os.path.basename(p)
        q.write_text(open(p).read())
        copies.append(str(q))
    base = kernel_code_hash(copies)
    assert base == kernel_code_hash()
    k = tmp_path / "fused_reduce_rmsnorm.hip"
    text = k.read_text()
    k.write_text("// a new comment line\n" + text.replace("\n", "\n  ", 3) + "\n/* trailing\n block */\n")
    assert kernel_code_hash(copies) == base                 # comments and layout only
    k.write_text(text.replace("__syncthreads();", "__syncthreads(); __syncthreads();", 1))
    assert kernel_code_hash(copies) != base                 # a code change
    k.write_text(text)
    g = tmp_path / "geometry.h"
    geo = g.read_text()
    g.write_text(geo.replace("{512, 2, 6, 2, 0}", "{512, 2, 5, 2, 0}"))
    assert kernel_code_hash(copies) != base                 # the geometry table is code too
    g.write_text(geo)
    from reduce_rmsnorm_amd.build import HIP_FLAGS, HIP_SOURCE_FLAGS
    flags = HIP_FLAGS + HIP_SOURCE_FLAGS["fused_reduce_rmsnorm.hip"]
    assert kernel_code_hash(copies, flags) == base
    assert kernel_code_hash(copies, HIP_FLAGS) != base      # so are its compile flags
