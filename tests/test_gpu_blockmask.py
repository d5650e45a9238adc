"""GPU parity of the dynamic block-mask generator (mad_block_mask) against the
oracle's pooled block scores and top-k, and of attention under a mask it made."""
import numpy as np
import pytest

import _gpu
from mad_inputs import qkv, variable_block_sizes
from oracle import attention as A
from oracle import blockscore as B
from oracle import masks as M

pytestmark = pytest.mark.gpu


def _edges(T, b, seed):
    if b == 0:
        s = variable_block_sizes(seed, T, 32, 256)
        return np.concatenate([[0], np.cumsum(s)]).astype(np.int32)
    return np.asarray(M.uniform_edges(T, b), dtype=np.int32)


def _run(q, k, qe, ke, G, pct, scale):
    import torch
    import mask_aware_dense_amd as mad
    dev = torch.device("cuda", 0)
    nqb, nkb = len(qe) - 1, len(ke) - 1
    Hkv, d = k.shape[1], k.shape[2]
    ws = torch.empty(mad.block_mask_workspace_bytes(G, Hkv, nqb, nkb, d), dtype=torch.uint8, device=dev)
    keep = torch.full((G, nqb, (nkb + 63) // 64), -1, dtype=torch.int64, device=dev)
    sc = torch.empty((G, nqb, nkb), dtype=torch.float32, device=dev)
    qe_d = torch.from_numpy(np.asarray(qe, np.int32)).to(dev)
    ke_d = torch.from_numpy(np.asarray(ke, np.int32)).to(dev)
    mad.block_mask(q.to(dev), k.to(dev), G, qe_d, ke_d, pct, scale, keep, ws, scores=sc)
    torch.cuda.synchronize()
    kw = keep.cpu().numpy().view(np.uint64)
    bits = np.zeros((G, nqb, nkb), dtype=bool)
    for j in range(nkb):
        bits[:, :, j] = (kw[:, :, j // 64] >> np.uint64(j % 64)) & np.uint64(1)
    pad = [(kw[:, :, j // 64] >> np.uint64(j % 64)) & np.uint64(1) for j in range(nkb, kw.shape[2] * 64)]
    return bits, sc.cpu().numpy(), kw, pad


@pytest.mark.parametrize("T,Hq,Hkv,G,d,b,pct", [
    (1000, 4, 2, 2, 128, 64, 50),     # GQA keep sets, ragged last block
    (2048, 4, 4, 4, 64, 64, 80),      # MHA, per-head keep sets
    (1500, 8, 2, 8, 128, 0, 20),      # per-head sets under GQA, variable blocks
    (4096, 8, 2, 2, 128, 128, 50),
    (300, 2, 1, 1, 64, 32, 100),      # k = 1
    (300, 2, 1, 2, 64, 32, 0),        # keep all
    (1200, 4, 2, 2, 256, 64, 50),     # head dim 256
])
def test_block_mask_matches_oracle(T, Hq, Hkv, G, d, b, pct):
    q, k, _ = qkv(T + pct, T, T, Hq, Hkv, d)
    qe = _edges(T, b, seed=T)
    ke = qe
    scale = 1.0 / np.sqrt(d)
    print(f"case block mask T={T} Hq={Hq} Hkv={Hkv} G={G} d={d} b={b} pct={pct}", flush=True)
    bits, sc, kw, pad = _run(q, k, qe, ke, G, pct, scale)
    ref = B.pooled_scores(q, k, qe, ke, G, scale)
    tol = 2e-5 * float(np.abs(ref).max()) + 1e-6
    err = float(np.abs(sc - ref).max())
    assert err <= tol, (err, tol)
    # the kernel's selection on its own fp32 scores: bit-exact
    assert np.array_equal(bits, M.topk_keep(sc, pct))
    assert all(int(x.max()) == 0 for x in pad) if pad else True
    # a valid top-k under the fp64 scores, up to the score tolerance
    nk = len(ke) - 1
    kk = max(1, nk - (pct * nk) // 100)
    assert np.all(bits.sum(axis=2) == kk)
    if kk < nk:
        lo = np.where(bits, ref, np.inf).min(axis=2)
        hi = np.where(~bits, ref, -np.inf).max(axis=2)
        assert np.all(lo >= hi - 2 * tol)


def test_attention_under_generated_mask():
    """Scores -> keep bitmap on the GPU -> plan -> attention forward and backward, against the oracle."""
    import mask_aware_dense_amd as mad
    T, Hq, Hkv, d, G = 1024, 4, 2, 128, 2
    q, k, v = qkv(77, T, T, Hq, Hkv, d)
    from mad_inputs import grad_out
    do = grad_out(77, T, Hq, d)
    e = _edges(T, 64, 0)
    scale = 1.0 / np.sqrt(d)
    bits, sc, kw, _ = _run(q, k, e, e, G, 50, scale)
    plan = mad.sparse_plan(G, e, e, kw)
    spec = M.MaskSpec("BLOCK_SPARSE", T, T, q_edges=e.astype(np.int64), k_edges=e.astype(np.int64), keep=bits)
    got = _gpu.gpu_attention(plan, q, k, v, do, scale)
    O, L = A.attn_fwd(q, k, v, spec, scale)
    g = A.attn_bwd(q, k, v, do, spec, scale)
    _gpu.check_close("o", got["o"], O, _gpu.TOL_FWD)
    _gpu.check_lse(got["lse"], L)
    for n in ("dq", "dk", "dv"):
        _gpu.check_close(n, got[n], g[n], _gpu.TOL_BWD)
