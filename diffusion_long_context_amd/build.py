"""Build ``libpdllm.so`` (the HIP kernels and the C ABI) in-tree for gfx950.

Every source under ``csrc/`` is compiled by ``hipcc`` for gfx950 only, in
parallel, and linked into ``diffusion_long_context_amd/libpdllm.so``.  The
library is replaced atomically so a running process keeps its mapping.

    python -m diffusion_long_context_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpdllm.so")
CALIB = os.path.join(HERE, "calib")
CALIB_LIB = os.path.join(HERE, "libpdllm_calib.so")   # peak calibration, measurement only
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed FP32 instructions
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(os.path.dirname(HERE), "include")]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpdllm")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 8, verbose: bool = False) -> str:
    """Compile every source and link the shared libraries (the path's
    libpdllm.so and the calibration libpdllm_calib.so); returns the path of
    libpdllm.so."""
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    calib = sorted(glob.glob(os.path.join(CALIB, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, sources + calib))
    _link(objs[:len(sources)], LIB)
    _link(objs[len(sources):], CALIB_LIB)
    if verbose:
        print(f"built {LIB} from {len(sources)} sources and {CALIB_LIB} from {len(calib)}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, jobs=int(sys.argv[1]) if len(sys.argv) > 1 else 8)
