"""Build libmad.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m mask_aware_dense_amd.build   (or call build()).
Always recompiles; objects go to mask_aware_dense_amd/_build/.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmad.so")
SOURCES = ["api.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_dkdv.hip", "ring.hip", "blockmask.hip", "plan_gpu.hip",
           "probe.hip", "mask_host.cpp"]
ARCH = os.environ.get("MAD_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def flags():
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5",
        # packed fp32 VALU forms stay off in every device build
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-Wno-unused-result",
        # MFMA results in arch VGPRs: the score tiles feed VALU softmax code
        # directly, and the register allocator then keeps every kernel
        # spill-free (measured: forward 58.9 -> 22.7 ms at 32K causal)
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        # the D = 256 step loops are longer than the default full-unroll
        # budget; partly unrolled, their operand arrays would be indexed at
        # run time (D = 64 / 128 code is the same either way)
        "-mllvm", "-pragma-unroll-threshold=1000000",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), *flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
