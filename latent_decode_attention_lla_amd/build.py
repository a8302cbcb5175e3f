"""Build the gfx950 HIP library ``liblla.so`` in-tree with hipcc.

Usage: python -m latent_decode_attention_lla_amd.build   (or __graft_entry__.build()).
Compiles every source under csrc/ for gfx950 on every call (hipcc cross-compiles, no GPU
needed) and links one shared library next to this file.

  python -m latent_decode_attention_lla_amd.build --asan
builds liblla_asan.so instead, with the host code (argument validation, planning, the
pointer arithmetic of the C ABI) under AddressSanitizer and the device code unchanged.
It is for CPU runs of the ABI tests only: load it by setting LLA_LIBRARY to its path and
preloading the ASan runtime (asan_runtime() names it), e.g.
  LD_PRELOAD=$(python -c 'from latent_decode_attention_lla_amd import build;
  print(build.asan_runtime())') ASAN_OPTIONS=detect_leaks=0 \
  LLA_LIBRARY=latent_decode_attention_lla_amd/liblla_asan.so python -m pytest tests/test_abi.py
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblla.so")
LIB_ASAN = os.path.join(HERE, "liblla_asan.so")
BUILD_ASAN = os.path.join(HERE, "_build_asan")
# host code only: each -fsanitize= follows -Xarch_host, so device code is not instrumented
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]

ARCH = "gfx950"
# Packed FP32 VALU forms are kept out of generated code (-packed-fp32-ops).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result"]
# Per-source additions. The narrow rotary-fold kernel and the reconstruct kernels are bound
# by vector-ALU issue; having their MFMA results written straight to VGPRs saves the
# AGPR-to-VGPR copies (five per 16-token tile for the fold, eight for a rebuilt tile)
# without raising their register counts.
_VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
FILE_FLAGS = {"decode_rotary_fold.hip": _VGPR_MFMA, "decode_reconstruct.hip": _VGPR_MFMA}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the LLA HIP library cannot be built")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def asan_runtime() -> str:
    """Path of the AddressSanitizer runtime that liblla_asan.so needs preloaded."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    return r.stdout.strip()


def build(verbose: bool = False, asan: bool = False) -> str:
    hipcc = _hipcc()
    build_dir = BUILD_ASAN if asan else BUILD
    lib_path = LIB_ASAN if asan else LIB
    extra = ASAN_FLAGS if asan else []
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIP_FLAGS, *extra, *FILE_FLAGS.get(os.path.basename(src), []), "-x", "hip",
               "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    jobs = min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = lib_path + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, asan="--asan" in sys.argv))
