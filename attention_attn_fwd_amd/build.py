"""Build the native parts of the package in-tree.

  libattn_fwd.so     hand-written HIP kernels for gfx950 + the C ABI
                     (csrc/*.hip, compiled with hipcc, one object per source,
                     in parallel, then linked)
  libattn_inputs.so  the seeded input generator (csrc/inputs.c, gcc + OpenMP)
  libattn_calib.so   a kernel of known MFMA count that calibrates the
                     hardware counters the benchmark reads (csrc/calib.hip;
                     loaded only by bench.py --workload mfma_cal)

Every HIP source is compiled with packed-fp32 instruction selection turned
off (-Xclang -target-feature -Xclang -packed-fp32-ops) and with MFMA results
kept in VGPRs (-mllvm -amdgpu-mfma-vgpr-form).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libattn_fwd.so")
INPUTS_LIB = os.path.join(HERE, "libattn_inputs.so")
CALIB_LIB = os.path.join(HERE, "libattn_calib.so")
ARCH = os.environ.get("ATTN_FWD_ARCH", "gfx950")

HIP_SOURCES = ["attn_api.hip", "prefill_bf16.hip", "decode_bf16.hip", "fwd_f32.hip", "bwd_bf16.hip"]
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the accumulators are also rescaled by
    # VALU code, and the AGPR form copies them back and forth every block.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build_lib(extra_flags=(), jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    headers = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    headers.append(os.path.join(ROOT, "include", "attn_fwd.h"))

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPCC_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        r = _run(cmd)
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs or min(len(HIP_SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, HIP_SOURCES))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def build_inputs() -> str:
    tmp = INPUTS_LIB + ".tmp"
    _run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
          "-o", tmp, os.path.join(CSRC, "inputs.c"), "-lm"])
    os.replace(tmp, INPUTS_LIB)
    return INPUTS_LIB


def build_calib() -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    obj = os.path.join(BUILD_DIR, "calib.o")
    _run([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, "calib.hip"), "-o", obj])
    tmp = CALIB_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj])
    os.replace(tmp, CALIB_LIB)
    return CALIB_LIB


def build_all(verbose: bool = False) -> list[str]:
    return [build_inputs(), build_lib(verbose=verbose), build_calib()]


if __name__ == "__main__":
    for p in build_all(verbose="-v" in sys.argv):
        print(p)
