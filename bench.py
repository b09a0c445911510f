"""Benchmark of the AVQ-Attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long-64k]

A step is one whole forward over one batch of synthetic inputs already
resident in HBM: stage 1 (avq_assign_aggregate: two kernels) then stage 2
(avq_attention_fwd: one kernel).  The frozen tree (avq_build_tree) is built
once before timing, as it is once per codebook.  Input sets rotate between
steps (4 sets, 768 MiB at the default workload) so that no step is served
from the 256 MiB Infinity Cache.

Prints ONE JSON line: the headline metric (tokens/s/head = B*N*H / step
time), the roofline of the dominant kernel measured with HIP events on the
stream the kernels run on, and the CPU oracle timed on a bounded sample on
this host's cores.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
# exponentials per second: 256 CUs x 4 SIMDs x 2.4 GHz, one wave64 v_exp_f32
# per 8 cycles per SIMD (measured issue cost) = 8 per cycle per SIMD
EXP_PEAK_PER_S = 256 * 4 * 2.4e9 * 8
MFMA_PEAK = {"bf16": 2500.0, "f32": 157.3}   # dense TFLOP/s (fp32 on the fp32 MFMA path)
METRIC = "AVQ attention fwd tokens/s/head at N=64k; % HBM BW and % MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(inp, P):
    """Algorithmic bytes and flops per launch ('Roofline')."""
    e = 2 if inp.dtype == "bf16" else 4
    BH, N, d, M0, C = inp.B * inp.H, inp.N, inp.d, inp.M0, inp.C
    S = M0 * (1 + C)
    s1_bytes = BH * (N * 2 * d * e + S * (4 * d + 4))
    s1_flops = BH * N * 2 * d * (M0 + C)
    s2_bytes = BH * (N * 2 * d * e + S * (4 * d + 4 + d * e))
    s2_flops = BH * N * 4 * d * (M0 + P * C)
    s2_exps = BH * N * (M0 + P * (C + 1))
    return dict(s1_bytes=s1_bytes, s1_flops=s1_flops, s2_bytes=s2_bytes, s2_flops=s2_flops,
                s2_exps=s2_exps)


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/traffic_<kernel>_<workload>.json), if it was taken on the
    current kernel source; else None."""
    from adaptive_vector_quantized_avq_amd import profiling
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        if rec.get("source_digest") != profiling.source_digest(kernel):
            return None
        return round(rec["bytes_per_launch"])
    except Exception:
        return None


def cpu_baseline(inp, P, heads):
    """The CPU oracle, as it stands, on the first `heads` heads of batch 0 of
    the workload: stage 1 on all their keys, stage 2 on all their query
    tiles."""
    import numpy as np
    import oracle
    import synth

    sub = synth.Inputs(**{**inp.__dict__})
    sub.B, sub.H = 1, heads
    sub.children = inp.children[:heads]
    sub.Q, sub.K, sub.V = (x[:1, :heads] for x in (inp.Q, inp.K, inp.V))
    ch = sub.f64("children")
    K64, V64, Q64 = sub.f64("K"), sub.f64("V"), sub.f64("Q")
    threads = oracle.default_threads()
    oracle.build_tree(ch[:1], inp.dtype)   # loads/compiles outside the timing
    t0 = time.perf_counter()
    par, _ = oracle.build_tree(ch, inp.dtype)
    a = oracle.assign(K64, par, ch, threads=threads)
    vsum, count = oracle.aggregate(V64, a["leaf"], inp.M0, inp.C, threads=threads)
    t1 = time.perf_counter()
    oracle.attention(Q64, par, ch, vsum, count, P, inp.T, inp.scale, threads=threads)
    t2 = time.perf_counter()
    tok = heads * inp.N
    return dict(value=tok / (t2 - t0), unit="tokens/s/head", cores=threads, kind="oracle",
                sample=f"{heads} of {inp.B * inp.H} (b,h) units of {inp.name}: stage 1 on all "
                       f"{inp.N} keys and stage 2 on all {inp.ntiles} query tiles of each, fp64",
                stage1_s=round(t1 - t0, 3), stage2_s=round(t2 - t1, 3))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long-64k")
    ap.add_argument("--P", type=int, default=None)
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads of batch 0 the CPU oracle runs on (0 = all of them)")
    ap.add_argument("--exact-context", action="store_true",
                    help="also time the in-repo exact softmax attention at the same shape")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy 5 times (a kernel of known "
                         "traffic, to calibrate the profiler's byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the method's "
              "multi-GPU split is described in DESIGN.md but not built", file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    import adaptive_vector_quantized_avq_amd as avq
    import synth

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    avq.load_library()

    inp = synth.generate(args.workload)
    P = inp.P if args.P is None else args.P
    log(f"workload {inp.name}: B={inp.B} H={inp.H} N={inp.N} d={inp.d} M0={inp.M0} C={inp.C} "
        f"P={P} T={inp.T} dtype={inp.dtype}")

    def to_dev(a):
        if inp.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    ch = to_dev(inp.children)
    Q0, K0, V0 = to_dev(inp.Q), to_dev(inp.K), to_dev(inp.V)
    # rotated copies: roll the token axis by whole query tiles (keys with
    # their values), so every set has the same statistics but other bytes
    sets = []
    for s in range(args.sets):
        sh = s * 7 * inp.T % inp.N
        sets.append(tuple(torch.roll(x, shifts=sh, dims=2).contiguous() for x in (Q0, K0, V0)))
    del Q0, K0, V0
    parents, sq = avq.build_tree(ch)
    B, H, N, d, S = inp.B, inp.H, inp.N, inp.d, inp.S_tot
    vsum = torch.empty((B, H, S, d), dtype=torch.float32, device=dev)
    count = torch.empty((B, H, S), dtype=torch.int32, device=dev)
    pack = torch.empty(avq.operand_pack_size(B, H, inp.M0, inp.C, d, sets[0][0].dtype),
                       dtype=torch.uint8, device=dev)
    ws = torch.empty(avq.assign_aggregate_workspace_size(B, H, N, inp.M0, inp.C, d),
                     dtype=torch.uint8, device=dev)
    Y = torch.empty_like(sets[0][0])

    def step(i, ev=None):
        Q, K, V = sets[i % len(sets)]
        if ev is not None:
            ev[0].record()
        avq.assign_aggregate(K, V, parents, ch, sq, workspace=ws, out=(vsum, count, pack))
        if ev is not None:
            ev[1].record()
        avq.attention_fwd(Q, parents, ch, pack, P, inp.T, inp.scale, out=Y)
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The K timed steps run back to back with events only around them (an
    # event between kernels is a marker the queue waits on, which would add
    # its own gap to every step).  The per-stage split comes from a second,
    # instrumented pass over K more steps right after it.
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record()
    for i in range(args.steps):
        step(i)
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span = e_start.elapsed_time(e_end)
    ms_step = span / args.steps

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    s1 = [e[0].elapsed_time(e[1]) for e in evs]
    s2 = [e[1].elapsed_time(e[2]) for e in evs]
    ms_step_instrumented = evs[0][0].elapsed_time(evs[-1][2]) / args.steps
    s1_ms, s2_ms = sum(s1) / len(s1), sum(s2) / len(s2)
    tokens = B * N * H
    value = tokens / (ms_step * 1e-3)

    alg = algorithmic(inp, P)
    peak_mf = MFMA_PEAK[inp.dtype]
    s1_gbs = alg["s1_bytes"] / (s1_ms * 1e-3) / 1e9
    s2_tfs = alg["s2_flops"] / (s2_ms * 1e-3) / 1e12
    s2_gbs = alg["s2_bytes"] / (s2_ms * 1e-3) / 1e9
    s2_bound = "mfma" if alg["s2_flops"] / (peak_mf * 1e12) >= alg["s2_bytes"] / (HBM_PEAK_GBS * 1e9) else "hbm"
    if s2_ms >= s1_ms:
        if s2_bound == "mfma":
            roof = dict(kernel="attention_kernel", bound="mfma", achieved=round(s2_tfs, 2),
                        peak=peak_mf, unit="TFLOP/s", frac=round(s2_tfs / peak_mf, 4))
        else:
            roof = dict(kernel="attention_kernel", bound="hbm", achieved=round(s2_gbs, 1),
                        peak=HBM_PEAK_GBS, unit="GB/s", frac=round(s2_gbs / HBM_PEAK_GBS, 4))
        roof["traffic"] = measured_traffic("attention_kernel", inp.name)
        roof["traffic_unit"] = "bytes per launch"
        roof["launch_ms"] = round(s2_ms, 5)
    else:
        t1 = measured_traffic("assign_parent_kernel", inp.name)
        t2 = measured_traffic("refine_aggregate_kernel", inp.name)
        roof = dict(kernel="assign_aggregate (assign_parent_kernel + refine_aggregate_kernel)", bound="hbm",
                    achieved=round(s1_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(s1_gbs / HBM_PEAK_GBS, 4),
                    traffic=(t1 + t2) if (t1 is not None and t2 is not None) else None,
                    traffic_unit="bytes per launch", launch_ms=round(s1_ms, 5))

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s/head",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic (seeded PCG64; shapes of the pages' long-sequence timing sweep)",
        "config": {"workload": inp.name, "B": B, "H": H, "N": N, "d": d, "M0": inp.M0,
                   "C": inp.C, "P": P, "tile": inp.T, "input_sets": args.sets},
        "roofline": roof,
        "stages": {
            "assign_aggregate": {"ms": round(s1_ms, 5), "alg_bytes": alg["s1_bytes"],
                                 "GBps": round(s1_gbs, 1), "frac_hbm": round(s1_gbs / HBM_PEAK_GBS, 4)},
            "attention_fwd": {"ms": round(s2_ms, 5), "alg_flops": alg["s2_flops"],
                              "alg_bytes": alg["s2_bytes"], "TFLOPs": round(s2_tfs, 2),
                              "GBps": round(s2_gbs, 1), "bound": s2_bound,
                              "frac_mfma": round(s2_tfs / peak_mf, 4),
                              "frac_hbm": round(s2_gbs / HBM_PEAK_GBS, 4),
                              "alg_exps": alg["s2_exps"],
                              "exp_bound_ms": round(alg["s2_exps"] / EXP_PEAK_PER_S * 1e3, 5)},
        },
        "host_wall_ms_per_step": round(wall / args.steps * 1e3, 5),
        "ms_per_step_with_stage_events": round(ms_step_instrumented, 5),
    }

    if args.exact_context:
        Q, K, V = sets[0]
        for _ in range(2):
            avq.exact_attention_fwd(Q, K, V, inp.scale, out=Y)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        reps = 3
        for _ in range(reps):
            avq.exact_attention_fwd(Q, K, V, inp.scale, out=Y)
        e1.record()
        torch.cuda.synchronize()
        ex_ms = e0.elapsed_time(e1) / reps
        out["exact_attention_context"] = {
            "ms": round(ex_ms, 4),
            "TFLOPs": round(4.0 * N * N * d * B * H / (ex_ms * 1e-3) / 1e12, 1),
            "speedup_avq": round(ex_ms / ms_step, 1)}

    if args.copy_probe:
        nbytes = 256 << 20
        xa = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_()
        ya = torch.empty_like(xa)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(5):
            ya.copy_(xa)
        c1.record()
        torch.cuda.synchronize()
        out["copy_probe"] = {"bytes_read": nbytes, "bytes_written": nbytes, "launches": 5,
                             "GBps": round(2 * nbytes * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9, 1)}

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        out["cpu_baseline"] = cpu_baseline(inp, P, max(1, min(args.cpu_heads or H, H)))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
