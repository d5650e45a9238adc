"""Element-wise parity of every output (O, LSE, dQ, dK, dV) on shapes whose dK/dV kernel runs with
one workgroup per key-tile column -- the form the benchmark times at CAUSAL 32K GQA 64:8: dK / dV
accumulated by one workgroup each and stored as bf16 directly, the group's shared visit list walked
from its end with the query heads innermost (GQA), the head-major variants (MHA with even columns)
and the 64-key two-wave tiling of 64-token blocks.  The split count is asserted, so these cases
cannot drift onto the cut-column path (fp32 partial sums), which the small parity cases take."""
import numpy as np
import pytest

import _gpu
import _pool
from mad_inputs import block_scores, grad_out, qkv
from oracle import masks as M

pytestmark = pytest.mark.gpu


def _run_and_check(plan, spec, Hq, Hkv, d, seed, heads, bn=None):
    import mask_aware_dense_amd as mad
    T = spec.Tq
    assert mad.bwd_kv_splits(plan, Hq, Hkv) == 1
    # -delta and -LSE/scale rows, then the kernels' 256 bytes of item-claim counters
    ws_one = (2 * Hq * ((T + 127) // 128 * 128) * 4 + 255) // 256 * 256 + 256
    assert mad.bwd_workspace_bytes(plan, T, T, Hq, Hkv, d) == ws_one  # no fp32 dK / dV sums
    if bn is not None:
        assert plan.info(1)["BN"] == bn
    q, k, v = qkv(seed, T, T, Hq, Hkv, d)
    do = grad_out(seed, T, Hq, d)
    scale = 1.0 / np.sqrt(d)
    print(f"case {spec.pattern} T={T} Hq={Hq} Hkv={Hkv} d={d} heads={list(heads)}", flush=True)
    got = _gpu.gpu_attention(plan, q, k, v, do, scale)
    ref = _pool.oracle_heads(q, k, v, do, spec, scale, heads)
    R = Hq // Hkv
    kvh = sorted({h // R for h in heads})
    assert all(set(range(g * R, (g + 1) * R)) <= set(heads) for g in kvh), "every head of a checked KV group"
    hs = list(heads)
    _gpu.check_close("o", got["o"][:, hs], ref["o"], _gpu.TOL_FWD)
    _gpu.check_lse(got["lse"][hs], ref["lse"])
    _gpu.check_close("dq", got["dq"][:, hs], ref["dq"], _gpu.TOL_BWD)
    _gpu.check_close("dk", got["dk"][:, kvh], ref["dk"][:, kvh], _gpu.TOL_BWD)
    _gpu.check_close("dv", got["dv"][:, kvh], ref["dv"][:, kvh], _gpu.TOL_BWD)


def test_causal_16k_gqa_16_8():
    """The benchmarked path at half length: CAUSAL, GQA with two query heads per KV head, d = 128;
    two KV heads (their four query heads) checked in full."""
    import mask_aware_dense_amd as mad
    T = 16384
    plan = mad.mask_compile(mad.mask_slices("CAUSAL", T), T, T)
    _run_and_check(plan, M.MaskSpec("CAUSAL", T, T), 16, 8, 128, seed=21, heads=[0, 1, 10, 11], bn=128)


@pytest.mark.parametrize("d", [128, 256])
def test_causal_4k_gqa_64_32(d):
    """CAUSAL 4K, GQA 64:32 (two query heads per KV head) at head dims 128 and 256 (the latter through
    the pair-of-waves dK/dV kernel, two 64-key workgroups per 128-key tile): every head checked."""
    import mask_aware_dense_amd as mad
    T = 4096
    plan = mad.mask_compile(mad.mask_slices("CAUSAL", T), T, T)
    _run_and_check(plan, M.MaskSpec("CAUSAL", T, T), 64, 32, d, seed=22, heads=range(64))


@pytest.mark.parametrize("d", [128, 256])
def test_full_4k_mha_16(d):
    """FULL 4K MHA 16:16: every visit list has one length, so the head-major kernels run."""
    import mask_aware_dense_amd as mad
    T = 4096
    plan = mad.mask_compile(mad.mask_slices("FULL", T), T, T)
    _run_and_check(plan, M.MaskSpec("FULL", T, T), 16, 16, d, seed=23, heads=range(16), bn=128)


def _sparse(T, b, G, pct, seed):
    import mask_aware_dense_amd as mad
    edges = np.asarray(M.uniform_edges(T, b), dtype=np.int32)
    n = len(edges) - 1
    scores = block_scores(seed, G, n, n)
    plan = mad.sparse_plan(G, edges, edges, mad.block_topk(scores, pct))
    spec = M.MaskSpec("BLOCK_SPARSE", T, T, q_edges=edges, k_edges=edges, keep=M.topk_keep(scores, pct))
    return plan, spec


@pytest.mark.parametrize("d", [128, 256])
def test_block_sparse_mha_8_b64_s80_8k(d):
    """Block-sparse MHA 8:8, 64-token blocks, 80% dropped: head-major 64-key dK/dV tiles (two-wave
    workgroups at d = 128, one pair-of-waves workgroup per tile at d = 256)."""
    plan, spec = _sparse(8192, 64, 8, 80, seed=24)
    _run_and_check(plan, spec, 8, 8, d, seed=24, heads=range(8), bn=64)


def test_block_sparse_gqa_16_8_b128_s50_16k():
    """Block-sparse GQA 16:8, 128-token blocks, half dropped: 128-key tiles, shared group lists."""
    plan, spec = _sparse(16384, 128, 8, 50, seed=25)
    _run_and_check(plan, spec, 16, 8, 128, seed=25, heads=[0, 1, 14, 15], bn=128)


def test_block_sparse_gqa_16_4_b64_s50_16k():
    """Block-sparse GQA 16:4, 64-token blocks, half dropped: 64-key two-wave tiles walked over a shared
    group list (four query heads per KV head)."""
    plan, spec = _sparse(16384, 64, 4, 50, seed=26)
    _run_and_check(plan, spec, 16, 4, 128, seed=26, heads=[4, 5, 6, 7], bn=64)
