"""Peak device memory of the path (LongCA-bench appendix A.4.2, the pages' second metric): the
forward's and the forward+backward's peaks equal the call's own tensors (inputs, outputs, backward
workspace, as the allocator counts their blocks) plus the plan's device block, and the free device
memory is the same before and after each call -- the kernels allocate nothing -- so the peak grows
linearly in T, where the pages' model of a standard attention module, 11bshd + 5bhs^2 + 2bshd,
grows with T^2."""
import os
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("mask,Hq,Hkv,kw", [("GLOBAL_SLIDING", 16, 16, {"global_len": 256, "window": 2048}),
                                           ("CAUSAL", 64, 8, {})])
def test_peak_equals_tensors_plus_plan(mask, Hq, Hkv, kw):
    import torch
    import mask_aware_dense_amd as mad
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench
    recs = {}
    for n, T in enumerate((2048, 2048, 8192)):
        print(f"case peak memory {mask} T={T} {Hq}:{Hkv}", flush=True)
        r = bench.peak_memory_case(torch, mad, mask, T, Hq, Hkv, 128, seed=0, kw=kw)
        print(r, flush=True)
        # the peak is the live tensors plus the plan: nothing transient is allocated by the calls
        assert r["fwd_peak_bytes"] == r["fwd_live_plus_plan_bytes"], r
        assert r["fwdbwd_peak_bytes"] == r["fwdbwd_live_plus_plan_bytes"], r
        # and the live blocks are the tensors themselves (the allocator rounds a block up by less than
        # a 2 MiB segment: 9 tensors at most)
        for ph in ("fwd", "fwdbwd"):
            extra = r[f"{ph}_peak_bytes"] - r[f"{ph}_tensors_plus_plan_bytes"]
            assert 0 <= extra <= 9 * (2 << 20), (ph, r)
        if n > 0:  # the first calls may load code objects; later ones must leave free memory unchanged
            assert r["free_bytes_change_fwd"] == 0 and r["free_bytes_change_bwd"] == 0, r
        recs[T] = r
    # tensors scale with T (the plan is a small O(tiles) term): 4x the tokens, at most ~4x the bytes,
    # while the standard-attention model grows ~16x
    ratio = recs[8192]["fwdbwd_peak_bytes"] / recs[2048]["fwdbwd_peak_bytes"]
    assert 3.9 < ratio < 4.2, ratio
    m = recs[8192]["standard_attention_activation_model_bytes"] / recs[2048]["standard_attention_activation_model_bytes"]
    assert m > 12, m
