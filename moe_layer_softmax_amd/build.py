"""Build libmoe.so (the gfx950 HIP library behind include/moe.h) in-tree with hipcc."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe.so")
# the HBM read-ceiling probe bench.py times (measurement only, a library of its own)
PROBE_LIB = os.path.join(HERE, "libmoe_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "route.hip", "permute.hip", "gemm.hip", "gemm_q.hip", "gemm_fp8.hip",
           "gemm_nv4.hip", "combine.hip", "quant.hip"]
# gemm_fp8.hip rescales every MFMA result with the vector ALU: its MFMAs are compiled in the form
# whose accumulators live in ordinary VGPRs (the default puts them in the MFMA-only registers,
# from which each result would need extra moves)
EXTRA = {"gemm_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
# Packed fp32 VALU ops are disabled for all device code (the compiler otherwise forms
# v_pk_{add,mul,fma}_f32 from ordinary float code).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(SRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    return obj


def build(jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    probe_obj = _compile("probe.hip")
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, probe_obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe link failed:\n" + r.stderr)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
