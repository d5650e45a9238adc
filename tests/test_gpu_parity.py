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


@pytest.mark.parametrize("d", [128, 64, 256])
@pytest.mark.parametrize("idx", range(len(M.STATIC_PATTERNS)))
def test_static_patterns_small(idx, d):
    T = 1000 + 37 * idx  # ragged: never a multiple of the 128 / 64 tile sizes
    spec = small_specs(T, seed=idx)[idx]
    _run_case(spec, _plan_for(spec), 8, 2, d, seed=100 + idx)


@pytest.mark.parametrize("bottom_right", [False, True])
@pytest.mark.parametrize("d", [128, 64, 256])
def test_varlen_cross_attention(bottom_right, d):
    """A batch of packed sequences with different query and key lengths (causal; bottom-right
    alignment leaves the first Lq - Lk rows of a sequence with no key: O = 0, LSE = -inf)."""
    import mask_aware_dense_amd as mad
    rng = np.random.default_rng(41 + d)
    lq, lk = rng.integers(1, 400, size=5), rng.integers(1, 400, size=5)
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    spec = M.MaskSpec("VARLEN", int(cq[-1]), int(ck[-1]), cu_q=tuple(int(x) for x in cq),
                      cu_k=tuple(int(x) for x in ck), causal=True, bottom_right=bottom_right)
    plan = mad.mask_compile(mad.varlen_slices(cq, ck, causal=True, bottom_right=bottom_right), spec.Tq, spec.Tk)
    _run_case(spec, plan, 8, 2, d, seed=300 + d + int(bottom_right))


def _sparse(T, b, G, pct, seed, variable):
    import mask_aware_dense_amd as mad
    if variable:
        edges = np.concatenate([[0], np.cumsum(variable_block_sizes(seed, T))]).astype(np.int64)
    else:
        edges = M.uniform_edges(T, b)
    n = len(edges) - 1
    scores = block_scores(seed, G, n, n)
    plan = mad.sparse_plan(G, edges, edges, mad.block_topk(scores, pct))
    spec = M.MaskSpec("VARIABLE_BLOCK_SPARSE" if variable else "BLOCK_SPARSE", T, T,
                      q_edges=edges, k_edges=edges, keep=M.topk_keep(scores, pct))
    return plan, spec


@pytest.mark.parametrize("b,variable", [(64, False), (128, False), (0, True)])
@pytest.mark.parametrize("pct", [20, 50, 80])
@pytest.mark.parametrize("heads", [(8, 8), (8, 2)], ids=["mha", "gqa"])
def test_block_sparse(b, variable, pct, heads):
    """Uniform 64/128 blocks and variable [32, 256] blocks; one keep set per KV head."""
    Hq, Hkv = heads
    T = 2048 if not variable else 1777
    plan, spec = _sparse(T, b, Hkv, pct, seed=pct + b + Hkv, variable=variable)
    _run_case(spec, plan, Hq, Hkv, 128, seed=7)


@pytest.mark.parametrize("b,variable", [(64, False), (0, True)])
@pytest.mark.parametrize("heads", [(8, 8), (8, 2)], ids=["mha", "gqa"])
def test_block_sparse_d256(b, variable, heads):
    """Head dim 256 (dK and dV from pairs of waves that each keep one 128-column half) under
    mixed-strip block masks."""
    Hq, Hkv = heads
    T = 1536 if not variable else 1333
    plan, spec = _sparse(T, b, Hkv, 50, seed=b + Hkv + 256, variable=variable)
    _run_case(spec, plan, Hq, Hkv, 256, seed=9)


def test_block_sparse_ragged_uniform():
    plan, spec = _sparse(1000, 64, 2, 50, seed=3, variable=False)  # last block of 40
    _run_case(spec, plan, 4, 2, 64, seed=8)


@pytest.mark.parametrize("layout", ["contiguous", "headtail"])
@pytest.mark.parametrize("rs", [(0, 0), (0, 7), (11, 3), (11, 11), (5, 9)])
def test_ring_step(layout, rs):
    """One rank's share of a 12-rank ring step at reduced chunk size (1024 tokens)."""
    r, s = rs
    C = 1024
    spec = M.MaskSpec("RING_STEP", C, C, layout=layout, n_ranks=12, rank=r, source=s)
    _run_case(spec, _plan_for(spec), 8, 1, 128, seed=20 + r * 12 + s)


def test_ring_step_d256():
    spec = M.MaskSpec("RING_STEP", 1024, 1024, layout="headtail", n_ranks=12, rank=5, source=9)
    _run_case(spec, _plan_for(spec), 8, 2, 256, seed=77)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("pattern", ["FULL", "CAUSAL"])
def test_forward_extreme_score_ranges(pattern, d):
    """Score ranges that the forward's lagging softmax reference must follow, one kind per query
    head: rising ramps along the keys, steep (300 log2 units per 64-key tile, so that p formed
    against the previous tile's reference overflows fp32) or mild (5 per tile, so that lane sums
    of p pass 2^8 without overflowing), falling ramps, and rows whose every score lies about 400
    log2 units below zero (p formed against a reference of 0 underflows to 0).  The oracle's
    softmax subtracts each row's exact max, so O and LSE are compared as in every other case.
    Forward only (the backward reads the forward's LSE and never forms a running max)."""
    torch = _gpu.torch_mod()
    T, Hq, Hkv = 1000, 8, 2
    q, k, v = qkv(17, T, T, Hq, Hkv, d)
    q, k = q.float(), k.float()
    k[:, :, 0] = (torch.arange(T, dtype=torch.float32) / 64)[:, None]  # one unit per 64-key tile
    k[:, :, 1] = 4.0
    unit = np.sqrt(d) / np.log2(np.e)  # a Q component of `unit` per unit of K adds one log2 unit
    ramp = [0, 300, 5, 0, -300, 5, 0, -5]       # log2 units per 64-key tile
    offset = [0, 0, 0, -400, 0, -400, 0, 0]     # log2 units on every score of the row
    for h in range(Hq):
        q[:, h, 0] = ramp[h] * unit
        q[:, h, 1] = offset[h] / 4 * unit
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    spec = M.MaskSpec(pattern, T, T)
    scale = 1.0 / np.sqrt(d)
    print(f"case extreme scores {pattern} T={T} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    got = _gpu.gpu_attention(_plan_for(spec), q, k, v, None, scale, bwd=False)
    O, L = A.attn_fwd(q, k, v, spec, scale)
    assert np.all(np.isfinite(L)) and L.max() > 2000 and L.min() < -200  # the ranges are as intended
    _gpu.check_close("o", got["o"], O, _gpu.TOL_FWD)
    _gpu.check_lse(got["lse"], L)


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("T", [1, 17, 65, 129])
def test_tiny_and_ragged(T, d):
    for pat in ("CAUSAL", "FULL"):
        spec = M.MaskSpec(pat, T, T)
        _run_case(spec, _plan_for(spec), 2, 1, d, seed=T)


def test_empty_key_range_gives_zero_and_neg_inf():
    """Tk = 0: every row has no allowed key -> O = 0, LSE = -inf, dQ = 0."""
    import mask_aware_dense_amd as mad
    plan = mad.mask_compile(np.zeros(0, dtype=mad.SLICE_DTYPE), 300, 0)
    q, _, _ = qkv(1, 300, 1, 4, 2, 128)
    k = q[:0, :2]
    got = _gpu.gpu_attention(plan, q, k, k, grad_out(1, 300, 4, 128), 0.1)
    assert np.all(got["o"] == 0) and np.all(np.isneginf(got["lse"])) and np.all(got["dq"] == 0)


@pytest.mark.parametrize("Tq,Tk,slices", [
    # keys 200..329 are seen by no row (a gap between a full and a causal slice)
    (300, 500, ((0, 300, 0, 200, 0, 0), (0, 300, 330, 500, 1, 0))),
    # no query rows at all: every key's dK, dV is 0
    (0, 300, ()),
])
def test_unseen_keys_get_zero_gradients(Tq, Tk, slices):
    """dK = dV = 0 are written for keys no query row sees, whatever the output buffers held
    before the calls (NaN here); the other outputs match the oracle."""
    import mask_aware_dense_amd as mad
    spec = M.MaskSpec("SLICES", Tq, Tk, slices=tuple(slices))
    arr = np.array(list(slices), dtype=mad.SLICE_DTYPE) if slices else np.zeros(0, dtype=mad.SLICE_DTYPE)
    plan = mad.mask_compile(arr, Tq, Tk)
    Hq, Hkv, d = 4, 2, 128
    q, k, v = qkv(11, Tq, Tk, Hq, Hkv, d)
    do = grad_out(11, Tq, Hq, d)
    scale = 1.0 / np.sqrt(d)
    print(f"case unseen keys Tq={Tq} Tk={Tk}", flush=True)
    got = _gpu.gpu_attention(plan, q, k, v, do, scale, fill=float("nan"))
    g = A.attn_bwd(q, k, v, do, spec, scale)
    seen = np.zeros(Tk, dtype=bool)
    for (q0, q1, k0, k1, _t, _w) in slices:
        seen[k0:k1] = q1 > q0
    assert np.all(got["dk"][~seen] == 0) and np.all(got["dv"][~seen] == 0)
    for n in ("dk", "dv"):
        _gpu.check_close(n, got[n], g[n], _gpu.TOL_BWD)
    if Tq:
        O, L = A.attn_fwd(q, k, v, spec, scale)
        _gpu.check_close("o", got["o"], O, _gpu.TOL_FWD)
        _gpu.check_lse(got["lse"], L)
        _gpu.check_close("dq", got["dq"], g["dq"], _gpu.TOL_BWD)


def test_rectangular_slices():
    """Tq != Tk with an arbitrary overlapping slice union."""
    import mask_aware_dense_amd as mad
    sl = [(0, 300, 0, 500, 1, 0), (100, 700, 200, 450, 0, 0), (650, 777, 600, 901, 1, 37)]
    spec = M.MaskSpec("SLICES", 777, 901, slices=tuple(sl))
    plan = mad.mask_compile(np.array(sl, dtype=mad.SLICE_DTYPE), 777, 901)
    _run_case(spec, plan, 4, 4, 128, seed=5)


@pytest.mark.parametrize("pattern", ["CAUSAL", "FULL_DOCUMENT"])
def test_forward_workspace_does_not_change_results(pattern):
    """With a workspace the forward's workgroups claim their items from per-XCD queues (the grid holds more
    workgroups than items); without one each takes a fixed item.  Each item is computed the same way
    either way, so O and LSE are bit-identical, and both match the oracle."""
    import torch
    import mask_aware_dense_amd as mad
    T, Hq, Hkv, d = 1100, 8, 2, 128
    docs = {"doc_lens": (300, 512, 288)} if pattern == "FULL_DOCUMENT" else {}
    spec = M.MaskSpec(pattern, T, T, **docs)
    plan = _plan_for(spec).upload()
    q, k, v = qkv(31, T, T, Hq, Hkv, d)
    dev = torch.device("cuda", 0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    fws = torch.empty(mad.FWD_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    outs = []
    for ws in (None, fws, fws):
        o = torch.full((T, Hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((Hq, T), float("nan"), dtype=torch.float32, device=dev)
        mad.attn_fwd(plan, qd, kd, vd, o, lse, 1 / np.sqrt(d), workspace=ws)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])
    O, L = A.attn_fwd(q, k, v, spec, 1 / np.sqrt(d))
    _gpu.check_close("o", outs[1][0].float().numpy(), O, _gpu.TOL_FWD)
    _gpu.check_lse(outs[1][1].numpy(), L)


def test_forward_workspace_errors():
    """A forward workspace shorter than FWD_WORKSPACE_BYTES is refused (MAD_ERR_INVALID) and so is one not
    256-byte aligned (MAD_ERR_UNSUPPORTED), before anything is launched: o and lse keep their contents."""
    import torch
    import mask_aware_dense_amd as mad
    T, Hq, Hkv, d = 256, 4, 2, 64
    plan = mad.mask_compile(mad.mask_slices("CAUSAL", T), T, T).upload()
    dev = torch.device("cuda", 0)
    q, k, v = (x.to(dev) for x in qkv(3, T, T, Hq, Hkv, d))
    o = torch.full((T, Hq, d), 7.0, dtype=torch.bfloat16, device=dev)
    lse = torch.full((Hq, T), 7.0, dtype=torch.float32, device=dev)
    buf = torch.empty(2 * mad.FWD_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    for ws, status in ((buf[:128], 1), (buf[16:16 + mad.FWD_WORKSPACE_BYTES], 2)):
        with pytest.raises(mad.MadError) as e:
            mad.attn_fwd(plan, q, k, v, o, lse, 0.125, workspace=ws)
        assert e.value.status == status, str(e.value)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())


def test_strided_inputs_and_determinism():
    """q, k, v as views of one fused [T, Hq + 2 Hkv, d] tensor; forward repeats bit for bit."""
    import torch
    import mask_aware_dense_amd as mad
    T, Hq, Hkv, d = 700, 4, 2, 128
    q, k, v = qkv(2, T, T, Hq, Hkv, d)
    dev = torch.device("cuda", 0)
    fused = torch.cat([q, k, v], dim=1).to(dev)
    qv, kv, vv = fused[:, :Hq], fused[:, Hq:Hq + Hkv], fused[:, Hq + Hkv:]
    spec = M.MaskSpec("CAUSAL", T, T)
    plan = _plan_for(spec).upload()
    outs = []
    for _ in range(2):
        o = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
        mad.attn_fwd(plan, qv, kv, vv, o, lse, 1 / np.sqrt(d))
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    O, L = A.attn_fwd(q, k, v, spec, 1 / np.sqrt(d))
    _gpu.check_close("o", outs[0][0].float().numpy(), O, _gpu.TOL_FWD)
    _gpu.check_lse(outs[0][1].numpy(), L)
