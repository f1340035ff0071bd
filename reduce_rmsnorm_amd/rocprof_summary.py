"""Turn rocprofv3 CSV output into the short summaries kept under profiles/.

Two subcommands:

``stats``    kernel_stats.csv of a ``--kernel-trace --stats`` run -> a
             markdown table of calls and durations.

``traffic``  counter_collection.csv of a ``--pmc FETCH_SIZE`` run and of a
             ``--pmc WRITE_SIZE`` run of ``bench.py --ceiling`` -> HBM bytes
             per launch of the fused kernel.  The counters are calibrated with
             the measurement probes of the same run: the read-only probe reads
             exactly (N+1) tensors and the write-only probe writes exactly 2,
             so the factor that turns each counter into bytes is known bytes
             over counted KiB*1024.  Writes a JSON (read by bench.py, keyed by
             the hash of the kernel source it was measured on) and a markdown
             note.

Usage (from the repo root)::

  python -m reduce_rmsnorm_amd.rocprof_summary stats RUN_kernel_stats.csv \
      --command "..." --out profiles/NAME.md
  python -m reduce_rmsnorm_amd.rocprof_summary traffic --fetch F.csv --write W.csv \
      --workload llama70b --command-fetch "..." --command-write "..." \
      --out profiles/NAME_traffic
"""

from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "reduce_rmsnorm_amd", "csrc")
# The fused kernel's code: its source and the headers it is built from.
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in
                  ("fused_reduce_rmsnorm.hip", "geometry.h", "device_common.h", "launch.h")]
FUSED = "fused_reduce_rmsnorm_kernel"
PROBE_READ = "probe_read<"
PROBE_WRITE = "probe_write("


def kernel_code_hash(paths=None, flags=None) -> str:
    """SHA-256 of the fused kernel's code with comments and whitespace
    removed, and of the flags it is compiled with: counters taken on one
    version stay attached to it through comment edits, and any change to the
    code itself (kernel, geometry table, device helpers) or to its compile
    flags gives a new hash.  (The sources hold no string literal containing
    comment markers.)"""
    h = hashlib.sha256()
    for path in paths or KERNEL_SOURCES:
        text = open(path, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(os.path.basename(path).encode())
        h.update(" ".join(text.split()).encode())
    if flags is None:
        from reduce_rmsnorm_amd.build import HIP_FLAGS, HIP_SOURCE_FLAGS
        flags = HIP_FLAGS + HIP_SOURCE_FLAGS.get(os.path.basename(KERNEL_SOURCES[0]), [])
    h.update(" ".join(flags).encode())
    return h.hexdigest()


def _medians(trace_path: str) -> dict:
    """Median dispatch duration (ns) per kernel name from a kernel_trace.csv."""
    durs = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_path)):
        durs[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = {}
    for name, v in durs.items():
        v.sort()
        n = len(v)
        out[name] = v[n // 2] if n % 2 else (v[n // 2 - 1] + v[n // 2]) / 2
    return out


def stats(path: str, command: str, out: str) -> None:
    rows = list(csv.DictReader(open(path)))
    # The per-dispatch trace of the same run, when present, gives the median.
    trace = path.replace("kernel_stats.csv", "kernel_trace.csv")
    med = _medians(trace) if trace != path and os.path.exists(trace) else {}
    lines = [f"# rocprofv3 kernel statistics: {os.path.basename(out)[:-3]}", "",
             "Command (run from /tmp with TMPDIR=/tmp, repo at $R):", "", "```", command, "```", "",
             "Kernel code sha256 (kernel source and headers with comments and whitespace removed, "
             f"and the compile flags): `{kernel_code_hash()}`", "",
             "| Kernel | Calls | Avg us | Median us | Min us | Max us | StdDev us | % time |",
             "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        m = med.get(r["Name"])
        lines.append("| `{}` | {} | {:.3f} | {} | {:.3f} | {:.3f} | {:.3f} | {:.2f} |".format(
            r["Name"], r["Calls"], float(r["AverageNs"]) / 1e3,
            "-" if m is None else f"{m / 1e3:.3f}", float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["StdDev"]) / 1e3, float(r["Percentage"])))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def _per_kernel(path: str, counter: str):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return agg


def _mean_of(agg, needle: str):
    vals = [v for k, vs in agg.items() if needle in k for v in vs]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {needle!r}")
    return sum(vals) / len(vals), len(vals)


def traffic(fetch: str, write: str, workload: str, cmd_fetch: str, cmd_write: str, out: str) -> None:
    sys.path.insert(0, ROOT)
    from synthetic import WORKLOADS
    wl = WORKLOADS[workload]
    tensor = wl.num_tokens * wl.hidden * wl.itemsize
    nsrc = wl.num_partials + 1
    fa, wa = _per_kernel(fetch, "FETCH_SIZE"), _per_kernel(write, "WRITE_SIZE")
    probe_fetch, n_pf = _mean_of(fa, PROBE_READ)
    probe_write, n_pw = _mean_of(wa, PROBE_WRITE)
    fused_fetch, n_ff = _mean_of(fa, FUSED)
    fused_write, n_fw = _mean_of(wa, FUSED)
    f_fetch = nsrc * tensor / (probe_fetch * 1024)
    f_write = 2 * tensor / (probe_write * 1024)
    read_b = fused_fetch * 1024 * f_fetch
    write_b = fused_write * 1024 * f_write
    alg = wl.algorithmic_bytes()
    res = {
        "kernel_code_sha256": kernel_code_hash(),
        "workload": f"{wl.name}: T={wl.num_tokens} h={wl.hidden} N={wl.num_partials} {wl.dtype}",
        "fetch_size_kib_per_launch": round(fused_fetch, 2),
        "write_size_kib_per_launch": round(fused_write, 2),
        "fetch_factor": round(f_fetch, 5),
        "write_factor": round(f_write, 5),
        "probe_read_fetch_kib": round(probe_fetch, 2),
        "probe_read_known_bytes": nsrc * tensor,
        "probe_write_write_kib": round(probe_write, 2),
        "probe_write_known_bytes": 2 * tensor,
        "read_bytes_per_launch": round(read_b),
        "write_bytes_per_launch": round(write_b),
        "bytes_per_launch": round(read_b + write_b),
        "algorithmic_bytes_per_launch": alg,
        "traffic_over_algorithmic": round((read_b + write_b) / alg, 5),
        "dispatches": {"fused_fetch": n_ff, "fused_write": n_fw, "probe_read": n_pf,
                       "probe_write": n_pw},
    }
    with open(out + ".json", "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    md = [f"# HBM traffic of the fused kernel, {res['workload']}", "",
          "Two counter passes of the same command (one counter each):", "", "```", cmd_fetch,
          cmd_write, "```", "",
          "Calibration with the measurement probes of the same runs:", "",
          f"- read-only probe: {nsrc} tensors x {tensor} B = {nsrc * tensor} B known, "
          f"FETCH_SIZE {probe_fetch:.1f} KiB per dispatch -> factor {f_fetch:.5f}",
          f"- write-only probe: 2 tensors x {tensor} B = {2 * tensor} B known, "
          f"WRITE_SIZE {probe_write:.1f} KiB per dispatch -> factor {f_write:.5f}", "",
          "Fused kernel, per launch (mean over dispatches):", "",
          "| | counter KiB | x factor = bytes | algorithmic bytes |", "|---|---|---|---|",
          f"| read | {fused_fetch:.1f} | {read_b:.0f} | {(wl.num_partials + 1) * tensor} |",
          f"| write | {fused_write:.1f} | {write_b:.0f} | {2 * tensor} |",
          f"| total | | {read_b + write_b:.0f} | {alg} |", "",
          f"Traffic / algorithmic bytes = {res['traffic_over_algorithmic']:.5f} "
          "(the weight row, 16 KiB, is fetched by each XCD's L2 and is not in the "
          "algorithmic count).", "",
          f"Kernel code sha256 (kernel source and headers with comments and whitespace removed, "
          f"and the compile flags): `{res['kernel_code_sha256']}`"]
    with open(out + ".md", "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(res, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--workload", default="llama70b")
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.cmd == "stats":
        stats(a.csv, a.command, a.out)
    else:
        traffic(a.fetch, a.write, a.workload, a.command_fetch, a.command_write, a.out)


if __name__ == "__main__":
    main()
