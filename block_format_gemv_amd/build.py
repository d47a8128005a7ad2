"""Build libqgemv.so (HIP, gfx950) in-tree: block_format_gemv_amd/libqgemv.so.

Every source under csrc/ is compiled by hipcc for --offload-arch=gfx950 with
-ffp-contract=off (no contraction of the exact f64/f32 steps), no fast-math and IEEE
denormal handling (but for the weighted sum's fold, kv_fold.hip, which flushes binary32
subnormals), and with packed-f32 instruction selection disabled; objects go to
_build/ and are linked into one shared library exporting the C ABI of include/qgemv.h.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "qgemv")
LIB = os.path.join(HERE, "libqgemv.so")
ARCH = os.environ.get("QG_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Werror",
          "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-fno-gpu-rdc",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# per-source device flags: the matrix-core GEMM keeps its MFMA accumulators in ordinary VGPRs
# (no copies out of AGPRs before the epilogue reads them); the weighted sum's fold runs with
# binary32 subnormals flushed (preserve-sign), the flushed add of its definition in hardware
EXTRA = {"gemm_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "kv_fold.hip": ["-fgpu-flush-denormals-to-zero"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    warn = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if warn.strip():
        sys.stderr.write(warn + "\n")
    return obj


def build(quiet: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if not quiet:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(quiet=False)
