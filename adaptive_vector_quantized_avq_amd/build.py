"""Compile the gfx950 HIP library (libavq.so) in-tree.

    python -m adaptive_vector_quantized_avq_amd.build

Every source under csrc/ is compiled with hipcc for gfx950 only, with packed
fp32 instructions disabled, into _build/, and linked into
adaptive_vector_quantized_avq_amd/libavq.so next to this file.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libavq.so")
PROBES = os.path.join(PKG, "probes")
PROBE_LIB = os.path.join(PKG, "libavq_peaks.so")   # throughput probes for bench.py --peaks
ARCH = "gfx950"


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas"]


# per-source extra flags:
#  -amdgpu-mfma-vgpr-form   keep MFMA results in VGPRs (no accumulator-register
#                           copies) where the VALU consumes every MFMA result;
#  -fno-honor-nans          every operand is finite by contract, so fminf /
#                           fmaxf lower to single v_min3 / v_max3 without NaN
#                           canonicalisation (the kernels' max3f / min3f)
EXTRA = {
    "assign_parent.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
    "refine_aggregate.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "attention_fwd.hip": ["-fno-honor-nans"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = EXTRA.get(os.path.basename(src), [])
    cmd = [_hipcc(), *COMMON, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    # the throughput probes are a separate library: bench.py loads them, the
    # AVQ library does not contain them
    psrc = os.path.join(PROBES, "peaks.hip")
    ptmp = PROBE_LIB + f".tmp{os.getpid()}"
    # (MFMA results in VGPRs: with accumulator registers the compiler copies
    # the eight accumulators through VGPRs every iteration, and the MFMA
    # probe then measures those copies)
    cmd = [_hipcc(), *COMMON, "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-shared", psrc, "-o", ptmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe library build failed:\n" + r.stdout + r.stderr)
    os.replace(ptmp, PROBE_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources, and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
