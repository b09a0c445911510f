"""Summaries of rocprofv3 output for the benchmark (text files under profiles/).

    python -m adaptive_vector_quantized_avq_amd.profiling kernels STATS_CSV CMD OUT_TXT
        per-kernel call count and mean duration from --kernel-trace --stats

    python -m adaptive_vector_quantized_avq_amd.profiling counters COUNTER_CSV CMD OUT_TXT
        per-kernel mean of every counter in one --pmc run (e.g. the SQ_*
        instruction and busy-cycle counters)

    python -m adaptive_vector_quantized_avq_amd.profiling traffic FETCH_CSV WRITE_CSV WORKLOAD CMD
        HBM bytes per launch of the stage kernels from two --pmc runs
        (FETCH_SIZE, then WRITE_SIZE), calibrated against the plain 256 MiB
        device copy that `bench.py --copy-probe` launches; writes
        profiles/traffic_<kernel>_<workload>.json (read by bench.py while the
        kernel source is unchanged) and a .txt summary beside it.

Only the parsing lives here; the counters come from the GPU runs whose full
command is recorded in each summary.
"""

from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")

# stage kernels and the sources their code comes from (for the digest that
# ties a traffic measurement to the kernel it was taken on)
_HDRS = ["adaptive_vector_quantized_avq_amd/csrc/avq_device.h",
         "adaptive_vector_quantized_avq_amd/csrc/avq_kernels.h"]
KERNEL_SOURCES = {
    "attention_kernel": ["adaptive_vector_quantized_avq_amd/csrc/attention_fwd.hip", *_HDRS],
    "pack_aggregates_kernel": ["adaptive_vector_quantized_avq_amd/csrc/pack_aggregates.hip", *_HDRS],
    "assign_parent_kernel": ["adaptive_vector_quantized_avq_amd/csrc/assign_parent.hip", *_HDRS],
    "refine_aggregate_kernel": ["adaptive_vector_quantized_avq_amd/csrc/refine_aggregate.hip", *_HDRS],
    "exact_attention_kernel": ["adaptive_vector_quantized_avq_amd/csrc/exact_attention.hip", *_HDRS],
    "bucket_children_kernel": ["adaptive_vector_quantized_avq_amd/csrc/tree3_stage1.hip", *_HDRS],
}
COPY_KERNEL = "probe_copy_kernel"   # the calibration copy (bench.py --copy-probe)
COPY_BYTES = 256 << 20        # bytes read and bytes written per copy launch


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    for k in KERNEL_SOURCES:
        if k in name:
            return k
    if COPY_KERNEL in name:
        return COPY_KERNEL
    return name.split("(")[0][:60]


def kernel_stats(path: str) -> dict:
    """{short name: (calls, mean ns)} from a rocprofv3 kernel_stats.csv."""
    out = {}
    for r in csv.DictReader(open(path)):
        out[short_name(r["Name"])] = (int(r["Calls"]), float(r["AverageNs"]))
    return out


def counter_means(path: str, counter: str) -> dict:
    """{short name: (dispatches, mean value)} of one counter."""
    acc = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"].startswith(counter):
            acc[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: (len(v), sum(v) / len(v)) for k, v in acc.items()}


def cmd_kernels(stats_csv: str, cmd: str, out_txt: str) -> None:
    st = kernel_stats(stats_csv)
    lines = [f"# rocprofv3 --kernel-trace --stats", f"# command: {cmd}", "",
             f"{'kernel':40s} {'calls':>6s} {'mean us':>10s}"]
    for k, (n, ns) in sorted(st.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        lines.append(f"{k:40s} {n:6d} {ns / 1e3:10.2f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_counters(csv_path: str, cmd: str, out_txt: str) -> None:
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(csv_path)):
        acc[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = ["# rocprofv3 --pmc (one pass; mean per dispatch)", f"# command: {cmd}", ""]
    for k in sorted(acc):
        lines.append(f"{k}  ({len(next(iter(acc[k].values())))} dispatches)")
        for c in sorted(acc[k]):
            v = acc[k][c]
            lines.append(f"  {c:32s} {sum(v) / len(v):16.1f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_traffic(fetch_csv: str, write_csv: str, workload: str, cmd: str) -> None:
    fetch = counter_means(fetch_csv, "FETCH_SIZE")
    write = counter_means(write_csv, "WRITE_SIZE")
    if COPY_KERNEL not in fetch or COPY_KERNEL not in write:
        raise SystemExit("no probe_copy_kernel dispatch in the counter files (run bench.py with --copy-probe)")
    # counters are in KiB per dispatch; scale so the copy reads and writes
    # exactly COPY_BYTES
    f_scale = COPY_BYTES / (fetch[COPY_KERNEL][1] * 1024.0)
    w_scale = COPY_BYTES / (write[COPY_KERNEL][1] * 1024.0)
    os.makedirs(PROFILES, exist_ok=True)
    for k in KERNEL_SOURCES:
        if k not in fetch or k not in write:
            continue
        rd = fetch[k][1] * 1024.0 * f_scale
        wr = write[k][1] * 1024.0 * w_scale
        rec = {"kernel": k, "workload": workload, "bytes_per_launch": rd + wr,
               "read_bytes": rd, "write_bytes": wr, "fetch_kib_raw": fetch[k][1],
               "write_kib_raw": write[k][1], "fetch_scale": f_scale, "write_scale": w_scale,
               "dispatches": [fetch[k][0], write[k][0]], "source_digest": source_digest(k),
               "command": cmd}
        base = os.path.join(PROFILES, f"traffic_{k}_{workload}")
        json.dump(rec, open(base + ".json", "w"), indent=1)
        txt = (f"# HBM traffic of {k} on {workload} (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)\n"
               f"# command (each counter in its own run): {cmd}\n"
               f"# calibration: the 256 MiB copy kernel reads {fetch[COPY_KERNEL][1]:.0f} KiB and writes "
               f"{write[COPY_KERNEL][1]:.0f} KiB per launch by the counters -> scale read x{f_scale:.3f}, "
               f"write x{w_scale:.3f}\n"
               f"read  {rd / 1e6:10.2f} MB per launch ({fetch[k][0]} dispatches)\n"
               f"write {wr / 1e6:10.2f} MB per launch ({write[k][0]} dispatches)\n"
               f"total {(rd + wr) / 1e6:10.2f} MB per launch\n")
        open(base + ".txt", "w").write(txt)
        print(txt)


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "kernels" and len(sys.argv) == 5:
        cmd_kernels(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 2 and sys.argv[1] == "counters" and len(sys.argv) == 5:
        cmd_counters(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 2 and sys.argv[1] == "traffic" and len(sys.argv) == 6:
        cmd_traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    else:
        print(__doc__)
        sys.exit(2)
