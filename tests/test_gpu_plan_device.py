"""GPU-compiled block-sparse plans (mad_sparse_plan_device) against the host
compiler: bit-identical visit lists, aux words, longest-first orders, pair and
tile counts, and the same attention outputs (O, LSE and dQ bit for bit)."""
import numpy as np
import pytest

import _gpu
from mad_inputs import block_scores, grad_out, qkv, variable_block_sizes
from oracle import masks as M

pytestmark = pytest.mark.gpu


def _edges(T, b, seed):
    if b == 0:
        s = variable_block_sizes(seed, T, 32, 256)
        return np.concatenate([[0], np.cumsum(s)]).astype(np.int32)
    return np.asarray(M.uniform_edges(T, b), dtype=np.int32)


def _keep_words(keep):
    """bool [G, nq, nk] -> uint64 [G, nq, ceil(nk/64)] (the bitmap layout)."""
    G, nq, nk = keep.shape
    out = np.zeros((G, nq, (nk + 63) // 64), dtype=np.uint64)
    for j in range(nk):
        out[:, :, j // 64] |= keep[:, :, j].astype(np.uint64) << np.uint64(j % 64)
    return out


def _both_plans(G, qe, ke, words):
    import torch
    import mask_aware_dense_amd as mad
    host = mad.sparse_plan(G, qe, ke, words)
    dev_keep = torch.from_numpy(words.view(np.int64)).to(torch.device("cuda", 0))
    devp = mad.sparse_plan_device(G, qe, ke, dev_keep)
    torch.cuda.synchronize()
    return host, devp


def _assert_same_plan(host, devp, G):
    for w in (0, 1):
        a, b = host.lists(w), devp.lists(w)
        for key in ("ptr", "ent", "ent_aux", "order"):
            assert np.array_equal(a[key], b[key]), (w, key)
        sa, sb = host.stats(w), devp.stats(w)
        assert np.array_equal(sa["pairs"], sb["pairs"])
        assert (sa["full"], sa["partial"], sa["empty"]) == (sb["full"], sb["partial"], sb["empty"])
        for g in sorted({0, G - 1}):
            ea, eb = host.export(w, g), devp.export(w, g)
            for key in ea:
                assert np.array_equal(ea[key], eb[key]), (w, g, key)


@pytest.mark.parametrize("Tq,Tk,G,bq,bk,pct", [
    (1000, 1000, 2, 64, 64, 50),      # ragged last block and tile
    (1000, 1000, 1, 128, 128, 20),
    (1500, 1500, 4, 0, 0, 80),        # variable blocks: PARTIAL tiles with mixed strips
    (2048, 2048, 8, 64, 64, 50),      # strips aligned to the blocks: aux words set
    (777, 1300, 3, 32, 96, 30),       # different query / key partitions
    (300, 300, 2, 32, 32, 100),       # one kept block per row
    (300, 300, 2, 32, 32, 0),         # everything kept
])
def test_device_plan_matches_host(Tq, Tk, G, bq, bk, pct):
    print(f"case plan_device Tq={Tq} Tk={Tk} G={G} bq={bq} bk={bk} pct={pct}", flush=True)
    qe, ke = _edges(Tq, bq, seed=Tq), _edges(Tk, bk, seed=Tk + 1)
    keep = M.topk_keep(block_scores(Tq + pct, G, len(qe) - 1, len(ke) - 1), pct)
    host, devp = _both_plans(G, qe, ke, _keep_words(keep))
    _assert_same_plan(host, devp, G)


def test_device_plan_ignores_bits_past_the_last_key_block():
    """Set bits beyond n_kb in the last bitmap word change nothing (as in the host compiler)."""
    T, G = 1000, 2
    qe = ke = _edges(T, 64, seed=3)
    keep = M.topk_keep(block_scores(5, G, len(qe) - 1, len(ke) - 1), 50)
    words = _keep_words(keep)
    dirty = words.copy()
    dirty[:, :, -1] |= ~np.uint64((1 << ((len(ke) - 1) % 64)) - 1)
    host, _ = _both_plans(G, qe, ke, words)
    _, devp = _both_plans(G, qe, ke, dirty)
    _assert_same_plan(host, devp, G)


@pytest.mark.parametrize("b,G,Hq,Hkv", [(64, 2, 4, 2), (0, 4, 4, 2)])
def test_attention_with_device_plan_is_bit_identical(b, G, Hq, Hkv):
    """The kernels read the same lists either way: O, LSE and dQ match bit for bit.  dK and dV
    of small problems are summed in fp32 over several workgroups per key tile (atomic adds in
    arrival order), so they agree to the last bits of a bf16 rounding only."""
    T, d = 1500, 128
    qe = ke = _edges(T, b, seed=9)
    keep = M.topk_keep(block_scores(11, G, len(qe) - 1, len(ke) - 1), 50)
    host, devp = _both_plans(G, qe, ke, _keep_words(keep))
    q, k, v = qkv(13, T, T, Hq, Hkv, d)
    do = grad_out(13, T, Hq, d)
    scale = 1.0 / np.sqrt(d)
    print(f"case plan_device attention b={b} G={G} Hq={Hq} Hkv={Hkv}", flush=True)
    a = _gpu.gpu_attention(host, q, k, v, do, scale, bwd=True)
    c = _gpu.gpu_attention(devp, q, k, v, do, scale, bwd=True)
    for key in ("o", "lse", "dq"):
        assert np.array_equal(a[key], c[key], equal_nan=True), key
    for key in ("dk", "dv"):
        x, y = a[key], c[key]
        assert np.all(np.abs(x - y) <= 2.0 ** -7 * np.abs(x) + 1e-6), key


def test_dynamic_mask_end_to_end_on_device():
    """Block scores and top-k on the GPU, then the plan compiled on the GPU from that bitmap:
    the same plan as the host compiler makes from the bitmap copied back."""
    import torch
    import mask_aware_dense_amd as mad
    T, Hq, Hkv, d, G, pct = 2048, 4, 2, 128, 2, 50
    dev = torch.device("cuda", 0)
    q, k, _ = qkv(21, T, T, Hq, Hkv, d)
    qe = ke = _edges(T, 64, seed=1)
    nqb, nkb = len(qe) - 1, len(ke) - 1
    ws = torch.empty(mad.block_mask_workspace_bytes(G, Hkv, nqb, nkb, d), dtype=torch.uint8, device=dev)
    keep = torch.empty((G, nqb, (nkb + 63) // 64), dtype=torch.int64, device=dev)
    qe_d = torch.from_numpy(qe).to(dev)
    ke_d = torch.from_numpy(ke).to(dev)
    mad.block_mask(q.to(dev), k.to(dev), G, qe_d, ke_d, pct, 1.0 / np.sqrt(d), keep, ws)
    devp = mad.sparse_plan_device(G, qe, ke, keep)
    torch.cuda.synchronize()
    host = mad.sparse_plan(G, qe, ke, keep.cpu().numpy().view(np.uint64))
    _assert_same_plan(host, devp, G)
