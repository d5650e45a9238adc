"""GPU parity at the largest sizes of the benchmark's configurations (block-sparse at 64K and
128K tokens, the dense document masks at 48K, MHA 64:64 and GQA 64:8), in the launch
configuration the benchmark times.  Inputs are drawn on the GPU; the oracle gets the sampled
heads' slices copied back and checks sampled rows of O, LSE and dQ; dK and dV are checked
through invariants that hold at any size (sum over keys of dK is 0; sum of dV equals the sum
of dO over rows that see at least one key)."""
import numpy as np
import pytest

import _gpu
from mad_inputs import block_scores, doc_lengths, grad_out_device, qkv_device, variable_block_sizes
from oracle import attention as A
from oracle import masks as M

pytestmark = pytest.mark.gpu


def _run(plan, q, k, v, do, scale):
    import torch
    import mask_aware_dense_amd as mad
    Tq, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    plan.upload()
    o = torch.empty_like(q)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    fws = torch.empty(mad.FWD_WORKSPACE_BYTES, dtype=torch.uint8, device=q.device)
    mad.attn_fwd(plan, q, k, v, o, lse, scale, workspace=fws)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(mad.bwd_workspace_bytes(plan, Tq, Tk, Hq, Hkv, d), 256), dtype=torch.uint8, device=q.device)
    mad.attn_bwd(plan, q, k, v, o, do, lse, dq, dk, dv, ws, scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _check(spec_for, q, k, v, do, out, heads, n_rows, seed, scale, n_groups):
    import torch
    o, lse, dq, dk, dv = out
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    rows = np.sort(np.random.default_rng(seed).choice(Tq, size=n_rows, replace=False))
    ridx = torch.from_numpy(rows).to(q.device)
    for h in heads:
        g, mg = h // (Hq // Hkv), h // (Hq // n_groups)
        sub = spec_for(mg)
        qs, ks, vs, ds = (t.cpu() for t in (q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], do[:, h:h + 1]))
        print(f"case xl head {h} (kv {g}, mask group {mg}) rows {n_rows}", flush=True)
        O, L = A.attn_fwd(qs, ks, vs, sub, scale, rows=rows)
        gq = A.attn_bwd(qs, ks, vs, ds, sub, scale, rows=rows, want=("dq",))["dq"]
        _gpu.check_close("o", o[ridx, h:h + 1].float().cpu().numpy(), O, _gpu.TOL_FWD)
        _gpu.check_lse(lse[h:h + 1][:, ridx].cpu().numpy().astype(np.float64), L)
        _gpu.check_close("dq", dq[ridx, h:h + 1].float().cpu().numpy(), gq, _gpu.TOL_BWD)
    # invariants over every key of every KV head (computed on the GPU in fp64); every row of
    # these masks sees at least one key
    R = Hq // Hkv
    sdk = dk.double().sum(dim=0)
    sdv = dv.double().sum(dim=0)
    ref = do.double().sum(dim=0).reshape(Hkv, R, d).sum(dim=1)
    for g in range(Hkv):
        nk = float(dk[:, g].double().norm())
        ndv = float(dv[:, g].double().norm())
        assert float(sdk[g].norm()) <= 1e-2 * nk, ("dk sum", g)
        assert float((sdv[g] - ref[g]).norm()) <= 1e-2 * max(ndv, 1.0), ("dv sum", g)


@pytest.mark.parametrize("S,Hq,Hkv,b,pct", [
    (131072, 64, 8, 128, 20),    # the largest block-sparse config, GQA
    (131072, 64, 64, 64, 80),    # MHA, per-head keep sets, 64-token blocks
    (65536, 64, 8, 0, 50),       # variable blocks
])
def test_block_sparse_largest(S, Hq, Hkv, b, pct):
    import torch
    import mask_aware_dense_amd as mad
    if b:
        edges = np.asarray(M.uniform_edges(S, b), dtype=np.int32)
    else:
        edges = np.concatenate([[0], np.cumsum(variable_block_sizes(7, S, 32, 256))]).astype(np.int32)
    n = len(edges) - 1
    G = Hkv  # one keep set per KV head (per head for MHA)
    keep = M.topk_keep(block_scores(S + pct, G, n, n), pct)
    words = np.zeros((G, n, (n + 63) // 64), dtype=np.uint64)
    for j in range(n):
        words[:, :, j // 64] |= keep[:, :, j].astype(np.uint64) << np.uint64(j % 64)
    print(f"case xl block-sparse S={S} Hq={Hq} Hkv={Hkv} b={b} pct={pct}", flush=True)
    plan = mad.sparse_plan_device(G, edges, edges, torch.from_numpy(words.view(np.int64)).cuda())
    q, k, v = qkv_device(S + 1, S, S, Hq, Hkv, 128)
    do = grad_out_device(S + 1, S, Hq, 128)
    scale = 1.0 / np.sqrt(128)
    out = _run(plan, q, k, v, do, scale)

    def spec_for(mg):
        return M.MaskSpec("VARIABLE_BLOCK_SPARSE" if not b else "BLOCK_SPARSE", S, S, q_edges=edges,
                          k_edges=edges, keep=keep[mg:mg + 1])
    _check(spec_for, q, k, v, do, out, heads=[0, Hq // 2 + 3, Hq - 1], n_rows=12, seed=S, scale=scale,
           n_groups=G)


@pytest.mark.parametrize("pattern,Hkv", [("CAUSAL_DOCUMENT", 64), ("SLIDING_WINDOW_CAUSAL_DOCUMENT", 8),
                                         ("FULL_DOCUMENT", 8)])
def test_document_masks_48k(pattern, Hkv):
    import mask_aware_dense_amd as mad
    T, Hq = 49152, 64
    docs = tuple(int(x) for x in doc_lengths(48, T))
    spec = M.MaskSpec(pattern, T, T, doc_lens=docs, window=4096)
    plan = mad.mask_compile(mad.mask_slices(pattern, T, **_gpu.spec_kwargs(spec)), T, T)
    print(f"case xl {pattern} T={T} Hq={Hq} Hkv={Hkv}", flush=True)
    q, k, v = qkv_device(T + Hkv, T, T, Hq, Hkv, 128)
    do = grad_out_device(T + Hkv, T, Hq, 128)
    scale = 1.0 / np.sqrt(128)
    out = _run(plan, q, k, v, do, scale)
    _check(lambda mg: spec, q, k, v, do, out, heads=[0, 37, 63], n_rows=12, seed=T, scale=scale, n_groups=1)
