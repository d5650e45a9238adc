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
SOURCES = ["api.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_dkdv.hip", "attn_dkdv256.hip", "ring.hip", "blockmask.hip",
           "plan_gpu.hip", "probe.hip", "mask_host.cpp"]
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


# Extra flags per source, each measured at CAUSAL 32K GQA 64:8 over
# alternating runs on one box.  The dQ kernel (attn_bwd.hip) is scheduled with
# the compiler's max-ILP strategy (dQ 21.43 -> 21.20 ms), the head-dim 64 /
# 128 dK/dV instances (attn_dkdv.hip) with iterative ILP scheduling (dK/dV
# 33.81 -> 33.48 ms).  The forward and the head-dim 256 dK/dV kernel
# (attn_dkdv256.hip, timed at CAUSAL 32K GQA 64:8 d=256) gained nothing from
# either.
SOURCE_FLAGS = {
    "attn_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "attn_dkdv.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


# Scratch (private memory) bytes per lane of every kernel, as validated by the
# GPU parity tests.  A kernel that spills registers adds scratch loads and
# stores to the vector-memory counter that the direct global->LDS copies are
# waited on with, so a changed register allocation must not slip in
# unnoticed: the build fails when any kernel's scratch size differs from its
# recorded value (0 for every kernel not listed; none spills now).
VALIDATED_SCRATCH: dict = {}


def _scratch_sizes(stderr: str) -> dict:
    """Kernel name -> ScratchSize [bytes/lane] from -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in stderr.splitlines():
        if "remark:" not in line:
            continue
        text = line.split("remark:", 1)[1].strip()
        if text.startswith("Function Name:"):
            cur = text.split(":", 1)[1].split()[0]
        elif text.startswith("ScratchSize") and cur is not None:
            out[cur] = int(text.split(":", 1)[1].split()[0])
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    hip = src.endswith(".hip")
    cmd = [hipcc(), *flags(), *SOURCE_FLAGS.get(src, []), *(["-Rpass-analysis=kernel-resource-usage"] if hip else []),
           "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if hip:
        sizes = _scratch_sizes(r.stderr)
        with open(os.path.join(CSRC, src)) as f:
            if "__global__" in f.read() and not sizes:
                raise RuntimeError(f"{src}: no kernel resource-usage remarks in the compiler output")
        bad = {k: v for k, v in sizes.items() if v != VALIDATED_SCRATCH.get(k, 0)}
        if bad:
            raise RuntimeError(f"{src}: kernel scratch sizes differ from the validated ones "
                               f"(bytes/lane): {bad}; expected {VALIDATED_SCRATCH} (others 0)")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    # -z defs: a reference no object defines fails the link instead of the load
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp,
           *objs, "-lpthread"]
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
