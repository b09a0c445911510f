"""bench.py's one-line JSON contract, on a small workload (GPU), and its
refusal of more than one GPU (CPU)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    sys.stdout.write(f"\n[case] bench.py {' '.join(args)}\n")
    sys.stdout.flush()
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=240)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, p.stdout
    return json.loads(lines[0])


@pytest.mark.gpu
def test_bench_json_line():
    pytest.importorskip("torch")
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = _run("--workload", "vit-b", "--steps", "3", "--warmup", "1", "--sets", "2", "--cpu-heads", "1")
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline", "oracle_check", "exact_baseline_ms"):
        assert k in d, k
    oc = d["oracle_check"]
    assert oc["max_abs_err"] is not None and oc["max_abs_err"] <= oc["tolerance"]
    assert oc["leaf_mismatch_outside_band"] == 0 and oc["selection_mismatch_outside_band"] == 0
    assert d["exact_baseline_ms"] > 0
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "vit-b" and d["dtype"] == "bf16"
    c = d["config"]
    assert abs(d["value"] - c["B"] * c["N"] * c["H"] / (d["ms_per_step"] * 1e-3)) <= 1e-3 * d["value"]
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma") and r["unit"] in ("GB/s", "TFLOP/s")
    assert 0 < r["achieved"] and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    b = d["cpu_baseline"]
    assert b["kind"] == "oracle" and b["value"] > 0 and b["cores"] >= 1


def test_bench_refuses_several_gpus():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode != 0 and "one GPU" in p.stderr
