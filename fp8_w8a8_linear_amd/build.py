"""Build libnhm.so (gfx950) in-tree with hipcc.

    python fp8_w8a8_linear_amd/build.py        # or __graft_entry__.build()

Every translation unit is compiled each time (a few seconds each, in parallel).
Packed-fp32 instruction selection is disabled for all device code.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libnhm.so")
ARCH = "gfx950"
SOURCES = ["api.hip", "quant.hip", "gemv.hip", "gemm.hip", "decode.hip", "norm.hip", "prefill.hip", "ssd.hip"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnhm)")


def flags():
    return ["-std=c++17", "-O3", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include")]


# Per-source flags. decode.hip: the compiler's atomic optimizer wraps the norm hand-off's
# counter increment in a wave-level aggregate whose result it reads right away, so the wave
# waited for the atomic's round trip before issuing the state stores meant to overlap it.
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, err in results:
        msgs = [ln for ln in err.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if verbose and msgs:
            print("\n".join(msgs), file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
