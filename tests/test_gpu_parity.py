"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small and mid sizes are compared element by element for every mask pattern;
sizes span several tiles of both tilings (128x64 and 64x128) and end in a
ragged tail.
"""
import numpy as np
import pytest

import _gpu
from _cases import small_specs
from mad_inputs import grad_out, qkv, doc_lengths, block_scores, variable_block_sizes
from oracle import attention as A
from oracle import masks as M

pytestmark = pytest.mark.gpu


def _plan_for(spec):
    import mask_aware_dense_amd as mad
    if spec.pattern in ("BLOCK_SPARSE", "VARIABLE_BLOCK_SPARSE"):
        raise AssertionError("use _sparse_plan")
    if spec.pattern == "RING_STEP":
        sl = mad.ring_step_slices(spec.layout, spec.n_ranks, spec.Tq, spec.rank, spec.source)
    else:
        sl = mad.mask_slices(spec.pattern, spec.Tq, **_gpu.spec_kwargs(spec))
    return mad.mask_compile(sl, spec.Tq, spec.Tk)


def _run_case(spec, plan, Hq, Hkv, d, seed, bwd=True):
    q, k, v = qkv(seed, spec.Tq, spec.Tk, Hq, Hkv, d)
    do = grad_out(seed, spec.Tq, Hq, d)
    scale = 1.0 / np.sqrt(d)
    print(f"case {spec.pattern} Tq={spec.Tq} Tk={spec.Tk} Hq={Hq} Hkv={Hkv} d={d} seed={seed}", flush=True)
    got = _gpu.gpu_attention(plan, q, k, v, do, scale, bwd=bwd)
    O, L = A.attn_fwd(q, k, v, spec, scale)
    _gpu.check_close("o", got["o"], O, _gpu.TOL_FWD)
    _gpu.check_lse(got["lse"], L)
    if bwd:
        g = A.attn_bwd(q, k, v, do, spec, scale)
        for n in ("dq", "dk", "dv"):
            _gpu.check_close(n, got[n], g[n], _gpu.TOL_BWD)


@pytest.mark.parametrize("pattern", ["FULL", "CAUSAL"])
def test_tiny_reference_config(pattern):
    """T=1024, MHA 4:4, d=64, FULL and CAUSAL, fwd + bwd in full."""
    spec = M.MaskSpec(pattern, 1024, 1024)
    _run_case(spec, _plan_for(spec), 4, 4, 64, seed=0)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("idx", range(12))
def test_static_patterns_small(idx, d):
    T = 1000 + 37 * idx  # ragged: never a multiple of the 128 / 64 tile sizes
    spec = small_specs(T, seed=idx)[idx]
    _run_case(spec, _plan_for(spec), 8, 2, d, seed=100 + idx)
