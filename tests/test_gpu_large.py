"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: sampled rows against the oracle, and backward invariants
that hold at any size for dK and dV (the oracle's dK/dV at these sizes would
need every row)."""
import numpy as np
import pytest

import _gpu
from mad_inputs import doc_lengths, grad_out, qkv
from oracle import attention as A
from oracle import masks as M

pytestmark = pytest.mark.gpu


def _full_run(spec, Hq, Hkv, d, seed, sl=None):
    import mask_aware_dense_amd as mad
    if sl is None:
        sl = mad.mask_slices(spec.pattern, spec.Tq, **_gpu.spec_kwargs(spec))
    plan = mad.mask_compile(sl, spec.Tq, spec.Tk)
    q, k, v = qkv(seed, spec.Tq, spec.Tk, Hq, Hkv, d)
    do = grad_out(seed, spec.Tq, Hq, d)
    scale = 1.0 / np.sqrt(d)
    print(f"case {spec.pattern} T={spec.Tq} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    got = _gpu.gpu_attention(plan, q, k, v, do, scale)
    return q, k, v, do, scale, got


def _check_sampled(spec, q, k, v, do, scale, got, n_rows=48, seed=0, heads=None):
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(spec.Tq, size=min(n_rows, spec.Tq), replace=False))
    Hq = q.shape[1]
    heads = list(range(Hq)) if heads is None else heads
    O, L = A.attn_fwd(q, k, v, spec, scale, rows=rows, heads=heads)
    g = A.attn_bwd(q, k, v, do, spec, scale, rows=rows, heads=heads, want=("dq",))
    _gpu.check_close("o", got["o"][rows][:, heads], O[:, heads], _gpu.TOL_FWD)
    _gpu.check_lse(got["lse"][heads][:, rows], L[heads])
    _gpu.check_close("dq", got["dq"][rows][:, heads], g["dq"][:, heads], _gpu.TOL_BWD)


def _check_bwd_invariants(got, do, nonempty, Hkv):
    """sum_j dK_j = 0 per KV head; sum_j dV_j = sum over rows with >= 1 key of dO (summed over the group)."""
    dk, dv = got["dk"], got["dv"]
    T, Hq, d = do.shape
    dof = do.float().numpy().astype(np.float64) * nonempty[:, :, None]
    ref_dv = dof.reshape(T, Hkv, Hq // Hkv, d).sum(axis=(0, 2))
    for g in range(Hkv):
        nk = np.linalg.norm(dk[:, g])
        print(f"kv head {g}: |sum dK|/|dK| = {np.linalg.norm(dk[:, g].sum(axis=0)) / nk:.2e}, "
              f"|sum dV - ref|/|dV| = {np.linalg.norm(dv[:, g].sum(axis=0) - ref_dv[g]) / np.linalg.norm(dv[:, g]):.2e}",
              flush=True)
        assert np.linalg.norm(dk[:, g].sum(axis=0)) <= 1e-2 * nk, ("dk sum", g)
        assert np.linalg.norm(dv[:, g].sum(axis=0) - ref_dv[g]) <= 1e-2 * max(np.linalg.norm(dv[:, g]), 1.0), ("dv sum", g)


def test_causal_32k_gqa_64_8():
    """The benchmarked workload: CAUSAL, T=32768, GQA 64:8, d=128."""
    spec = M.MaskSpec("CAUSAL", 32768, 32768)
    q, k, v, do, scale, got = _full_run(spec, 64, 8, 128, seed=0)
    _check_sampled(spec, q, k, v, do, scale, got, n_rows=32, heads=[0, 7, 8, 33, 63])
    _check_bwd_invariants(got, do, np.ones((32768, 64), bool), 8)


def test_causal_16k_gqa_64_8_d256():
    """Head dim 256 at a full size: CAUSAL, T=16384, GQA 64:8 (dK, dV from pairs of waves that each
    keep one column half)."""
    spec = M.MaskSpec("CAUSAL", 16384, 16384)
    q, k, v, do, scale, got = _full_run(spec, 64, 8, 256, seed=4)
    _check_sampled(spec, q, k, v, do, scale, got, n_rows=24, heads=[0, 9, 40, 63])
    _check_bwd_invariants(got, do, np.ones((16384, 64), bool), 8)


def test_global_sliding_32k_gqa_64_8():
    """GLOBAL_SLIDING at the suite's shape (256 global keys, 2K window): its two global key tiles
    hold most of the dK/dV items, so their columns are cut between workgroups (fp32 sums)."""
    T = 32768
    spec = M.MaskSpec("GLOBAL_SLIDING", T, T, global_len=256, window=2048)
    q, k, v, do, scale, got = _full_run(spec, 64, 8, 128, seed=6)
    _check_sampled(spec, q, k, v, do, scale, got, n_rows=24, heads=[0, 13, 63])
    _check_bwd_invariants(got, do, np.ones((T, 64), bool), 8)


def test_block_sparse_32k_gpu_plan():
    """Block-sparse 32K GQA 64:8, b=128, half the key blocks dropped, with the plan compiled on
    the GPU from a device keep bitmap: sampled rows against the oracle."""
    import torch
    import mask_aware_dense_amd as mad
    from mad_inputs import block_scores
    T, b, G = 32768, 128, 8
    edges = np.asarray(M.uniform_edges(T, b), dtype=np.int32)
    n = len(edges) - 1
    keep = M.topk_keep(block_scores(17, G, n, n), 50)
    plan = mad.sparse_plan(G, edges, edges, mad.block_topk(block_scores(17, G, n, n), 50))
    words = np.zeros((G, n, (n + 63) // 64), dtype=np.uint64)
    for j in range(n):
        words[:, :, j // 64] |= keep[:, :, j].astype(np.uint64) << np.uint64(j % 64)
    dplan = mad.sparse_plan_device(G, edges, edges, torch.from_numpy(words.view(np.int64)).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(plan.lists(0)["ent"], dplan.lists(0)["ent"])
    spec = M.MaskSpec("BLOCK_SPARSE", T, T, q_edges=edges, k_edges=edges, keep=keep)
    q, k, v = qkv(17, T, T, 64, 8, 128)
    do = grad_out(17, T, 64, 128)
    scale = 1.0 / np.sqrt(128)
    print("case BLOCK_SPARSE 32K GQA 64:8 b128 s0.5 (GPU plan)", flush=True)
    got = _gpu.gpu_attention(dplan, q, k, v, do, scale)
    _check_sampled(spec, q, k, v, do, scale, got, n_rows=16, seed=5, heads=[0, 9, 63])
    _check_bwd_invariants(got, do, np.ones((T, 64), bool), 8)


@pytest.mark.parametrize("pattern", ["SLIDING_WINDOW_CAUSAL_DOCUMENT", "SHARED_QUESTION", "BLOCK_CAUSAL_DOCUMENT",
                                     "CAUSAL_BLOCKWISE_LAST", "BLOCK_CAUSAL_DOCUMENT_GLOBAL"])
def test_16k_workload_masks(pattern):
    T = 16384
    docs = tuple(int(x) for x in doc_lengths(11, T))
    spec = M.MaskSpec(pattern, T, T, doc_lens=docs, window=4096, block=1024)
    q, k, v, do, scale, got = _full_run(spec, 16, 2, 128, seed=3)
    _check_sampled(spec, q, k, v, do, scale, got, n_rows=24)
    _check_bwd_invariants(got, do, np.ones((T, 16), bool), 2)


def test_ring_step_full_shape():
    """A head-tail ring step at its real shape: 8K local queries x 8K remote keys, GQA 64:8."""
    import mask_aware_dense_amd as mad
    C = 8192
    spec = M.MaskSpec("RING_STEP", C, C, layout="headtail", n_ranks=12, rank=0, source=0)
    sl = mad.ring_step_slices("headtail", 12, C, 0, 0)
    q, k, v, do, scale, got = _full_run(spec, 64, 8, 128, seed=4, sl=sl)
    _check_sampled(spec, q, k, v, do, scale, got, n_rows=24, heads=[0, 9, 63])


def _check_keys(spec, q, k, v, do, scale, got, kv_head, keys):
    """dK / dV of one KV head at chosen key columns, element by element against the oracle (every
    query row of the group's heads that sees one of the keys; process pool over those heads)."""
    import _pool
    dk, dv = _pool.oracle_keys(q, k, v, do, spec, scale, keys, kv_head)
    _gpu.check_close("dk", got["dk"][keys, kv_head], dk, _gpu.TOL_BWD)
    _gpu.check_close("dv", got["dv"][keys, kv_head], dv, _gpu.TOL_BWD)


@pytest.mark.parametrize("pattern", ["FULL", "SLIDING_WINDOW", "PREFIX_LM", "CAUSAL_BLOCKWISE", "PREFIX_LM_DOCUMENT"])
def test_32k_gqa_64_8_patterns(pattern):
    """Static patterns at the suite's 32K GQA 64:8 shape and parameters (4K window, 25% prefix, 2K
    blocks, documents log-uniform in [512, 16K]): sampled rows of O, LSE, dQ, and dK / dV of one KV
    head at sampled keys (tile edges, the first and last key, and random ones)."""
    T = 32768
    docs = tuple(int(x) for x in doc_lengths(13, T))
    spec = M.MaskSpec(pattern, T, T, window=4096, block=2048, doc_lens=docs)
    q, k, v, do, scale, got = _full_run(spec, 64, 8, 128, seed=31)
    _check_sampled(spec, q, k, v, do, scale, got, n_rows=24, seed=3, heads=[0, 21, 63])
    rng = np.random.default_rng(7)
    keys = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 8191, 8192, 16383, 32767],
                                     rng.choice(T, size=6, replace=False)]))
    _check_keys(spec, q, k, v, do, scale, got, kv_head=5, keys=keys)
    _check_bwd_invariants(got, do, np.ones((T, 64), bool), 8)
