"""GPU parity of the LSE merge and of one rank's share of ring context
parallelism (the ring object), against the oracle: the merge against the
merge formula on the same bf16 parts, and the ring against dense causal
attention over the whole sequence restricted to the rank's rows."""
import numpy as np
import pytest

import _gpu
from mad_inputs import grad_out, qkv
from oracle import attention as A
from oracle import masks as M
from oracle import merge as MG

pytestmark = pytest.mark.gpu


def _rank_rows(layout, N, C, rank):
    """Global sequence rows held by `rank`, in local order."""
    loc = np.arange(C)
    spec = M.MaskSpec("RING_STEP", C, C, layout=layout, n_ranks=N, rank=rank, source=rank)
    return M._ring_positions(spec, loc, "q")


@pytest.mark.parametrize("d,n", [(128, 3), (64, 5), (128, 1), (256, 4)])
def test_lse_merge(d, n):
    """Merge of n bf16 partial outputs: rows with every part -inf, rows with some -inf parts."""
    import torch
    import mask_aware_dense_amd as mad
    rng = np.random.default_rng([n, d])
    Tq, Hq = 203, 3
    o_parts = [rng.standard_normal((Tq, Hq, d)) for _ in range(n)]
    lse_parts = [rng.normal(2.0, 3.0, size=(Hq, Tq)) for _ in range(n)]
    for t in range(n):
        drop = rng.random((Hq, Tq)) < 0.3
        lse_parts[t][drop] = -np.inf
    lse_parts[0][:, :7] = -np.inf
    for t in range(n):
        lse_parts[t][:, 3] = -np.inf  # a row with no keys in any part
    ob = [torch.tensor(x, dtype=torch.float32).to(torch.bfloat16) for x in o_parts]
    lb = [torch.tensor(x, dtype=torch.float32) for x in lse_parts]
    ref_o, ref_l = MG.merge([x.float().numpy() for x in ob], [x.numpy() for x in lb])
    dev = torch.device("cuda", 0)
    od = [x.to(dev) for x in ob]
    ld = [x.to(dev) for x in lb]
    o = torch.empty((Tq, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=dev)
    print(f"case merge d={d} n={n}", flush=True)
    mad.lse_merge(od, ld, o, lse)
    torch.cuda.synchronize()
    _check_merged("o", o.float().cpu().numpy(), ref_o)
    _gpu.check_lse(lse.cpu().numpy(), ref_l)
    assert np.all(o.float().cpu().numpy()[3] == 0.0)
    # in place: the output aliases part 0
    mad.lse_merge(od, ld, od[0], ld[0])
    torch.cuda.synchronize()
    _check_merged("o in place", od[0].float().cpu().numpy(), ref_o)


def _check_merged(name, got, ref):
    """The merged O is computed in fp32 and rounded once to bf16, which moves a value by at most
    2^-8 of its magnitude (half an ulp of an 8-bit significand); 1e-4 covers the fp32 sums."""
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4
    assert np.all(err <= bound), f"{name}: worst excess {float((err - bound).max()):.3e}"
    _gpu.check_close(name, got, ref, (2e-2, 5e-3))


def _ring_case(layout, N, C, rank, Hq, Hkv, d, seed, rows_check=None, full_bwd=True):
    import torch
    import mask_aware_dense_amd as mad
    T = N * C
    q, k, v = qkv(seed, T, T, Hq, Hkv, d)
    do = grad_out(seed, T, Hq, d)
    g_rows = _rank_rows(layout, N, C, rank)
    dev = torch.device("cuda", 0)
    ql = q[torch.from_numpy(g_rows)].contiguous().to(dev)
    dol = do[torch.from_numpy(g_rows)].contiguous().to(dev)
    kd, vd = k.to(dev), v.to(dev)
    scale = 1.0 / np.sqrt(d)
    ring = mad.Ring(layout, N, C, rank, Hq, Hkv, d)
    o = torch.empty((C, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Hq, C), dtype=torch.float32, device=dev)
    dq = torch.empty_like(ql)
    dk = torch.full_like(kd, 7.0)
    dv = torch.full_like(vd, 7.0)
    print(f"case ring {layout} N={N} C={C} rank={rank} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    ring.fwd(ql, kd, vd, o, lse, scale)
    ring.bwd(ql, kd, vd, o, dol, lse, dq, dk, dv, scale)
    torch.cuda.synchronize()
    got = {"o": o.float().cpu().numpy(), "lse": lse.cpu().numpy(), "dq": dq.float().cpu().numpy(),
           "dk": dk.float().cpu().numpy(), "dv": dv.float().cpu().numpy()}
    info = ring.info()
    del ring
    return q, k, v, do, g_rows, scale, got, info


@pytest.mark.parametrize("layout,rank,d", [("contiguous", 0, 128), ("contiguous", 2, 128), ("contiguous", 3, 128),
                                           ("headtail", 0, 128), ("headtail", 2, 128), ("headtail", 3, 128),
                                           ("headtail", 1, 256)])
def test_ring_small(layout, rank, d):
    """Whole share of a 4-rank ring at chunk 256: merged O/LSE, accumulated dQ and the rank's dK/dV share."""
    N, C, Hq, Hkv = 4, 256, 4, 2
    q, k, v, do, g_rows, scale, got, info = _ring_case(layout, N, C, rank, Hq, Hkv, d, seed=rank + 11)
    spec = M.MaskSpec("CAUSAL", N * C, N * C)
    O, L = A.attn_fwd(q, k, v, spec, scale, rows=g_rows)
    g = A.attn_bwd(q, k, v, do, spec, scale, rows=g_rows)
    _gpu.check_close("o", got["o"], O, _gpu.TOL_FWD)
    _gpu.check_lse(got["lse"], L)
    _gpu.check_close("dq", got["dq"], g["dq"], _gpu.TOL_BWD)
    _gpu.check_close("dk", got["dk"], g["dk"], _gpu.TOL_BWD)
    _gpu.check_close("dv", got["dv"], g["dv"], _gpu.TOL_BWD)
    pairs = int(M.allowed(spec, g_rows, np.arange(N * C)).sum())
    assert info["pairs_per_head"] == pairs


@pytest.mark.parametrize("layout,rank", [("headtail", 0), ("contiguous", 11)])
def test_ring_full_shape(layout, rank):
    """One rank of the 12-rank ring at its real shape (8K chunks, GQA 64:8, d=128): sampled rows
    against dense causal attention over the 96K sequence, and backward invariants for dK/dV."""
    N, C, Hq, Hkv, d = 12, 8192, 64, 8, 128
    q, k, v, do, g_rows, scale, got, info = _ring_case(layout, N, C, rank, Hq, Hkv, d, seed=5)
    rng = np.random.default_rng(rank)
    loc = np.sort(rng.choice(C, size=24, replace=False))
    heads = [0, 9, 63]
    spec = M.MaskSpec("CAUSAL", N * C, N * C)
    O, L = A.attn_fwd(q, k, v, spec, scale, rows=g_rows[loc], heads=heads)
    gq = A.attn_bwd(q, k, v, do, spec, scale, rows=g_rows[loc], heads=heads, want=("dq",))
    _gpu.check_close("o", got["o"][loc][:, heads], O[:, heads], _gpu.TOL_FWD)
    _gpu.check_lse(got["lse"][heads][:, loc], L[heads])
    _gpu.check_close("dq", got["dq"][loc][:, heads], gq["dq"][:, heads], _gpu.TOL_BWD)
    # sum_j dK_j = 0 per KV head (sum_j dS_ij = 0 for every row), and
    # sum_j dV_j = the group's sum of dO over the rank's rows (each has >= 1 key).
    dof = do.float().numpy().astype(np.float64)[g_rows]
    ref_dv = dof.reshape(C, Hkv, Hq // Hkv, d).sum(axis=(0, 2))
    for gk in range(Hkv):
        nk = np.linalg.norm(got["dk"][:, gk])
        assert np.linalg.norm(got["dk"][:, gk].sum(axis=0)) <= 1e-2 * nk, ("dk sum", gk)
        assert np.linalg.norm(got["dv"][:, gk].sum(axis=0) - ref_dv[gk]) <= 1e-2 * np.linalg.norm(got["dv"][:, gk])
    n_steps = info["n_steps"]
    assert n_steps == 12
