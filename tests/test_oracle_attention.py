"""Pins for the fp64 oracle's attention forward and backward.

Each test checks the oracle against something other than itself: a
pure-Python brute force, a hand-derived fixture, a closed form, torch's
scaled_dot_product_attention in fp64 (a library routine on the unmasked or
boolean-masked case), central finite differences, or an invariant of softmax
attention.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import _brute
from _cases import small_specs, sparse_spec
from mad_inputs import variable_block_sizes
from oracle import attention as A
from oracle import masks as M

HERE = os.path.dirname(os.path.abspath(__file__))


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def nested(x):
    return x.tolist()


def all_tiny_specs(T):
    specs = small_specs(T, seed=3)
    specs.append(sparse_spec(T, 4, 2, 50, seed=1))
    specs.append(sparse_spec(T, 4, 2, 50, seed=2, variable_sizes=variable_block_sizes(5, T, lo=2, hi=7)))
    for layout in ("contiguous", "headtail"):
        for s in range(3):
            specs.append(M.MaskSpec("RING_STEP", T, T, layout=layout, n_ranks=3, rank=1, source=s))
    return specs


def _allowed_fn(spec, Hq):
    def f(h, i, j):
        G = spec.n_groups
        mg = h // (Hq // G) if G > 1 else 0
        return bool(M.allowed(spec, [i], [j], mg)[0, 0])
    return f


N_TINY = len(all_tiny_specs(16))


def test_every_tiny_spec_is_brute_forced():
    """The brute-force tests below cover every tiny spec, at both sizes."""
    assert N_TINY == len(all_tiny_specs(24)) == 22


@pytest.mark.parametrize("idx", range(N_TINY))
def test_fwd_matches_brute_force(idx):
    T, Hq, Hkv, d = 24, 4, 2, 5
    spec = all_tiny_specs(T)[idx]
    q, k, v = rnd(idx, T, Hq, d), rnd(100 + idx, T, Hkv, d), rnd(200 + idx, T, Hkv, d)
    scale = 0.7
    O, L = A.attn_fwd(q, k, v, spec, scale)
    Ob, Lb = _brute.fwd(nested(q), nested(k), nested(v), _allowed_fn(spec, Hq), scale)
    Ob, Lb = np.array(Ob), np.array(Lb)
    assert np.array_equal(np.isinf(L), np.isinf(Lb)), spec.pattern
    assert np.max(np.abs(O - Ob)) < 1e-12, spec.pattern
    fin = np.isfinite(L)
    assert np.max(np.abs(L[fin] - Lb[fin]), initial=0.0) < 1e-12, spec.pattern


@pytest.mark.parametrize("idx", range(N_TINY))
def test_bwd_matches_brute_force(idx):
    T, Hq, Hkv, d = 16, 4, 2, 3
    spec = all_tiny_specs(T)[idx]
    q, k, v, do = rnd(idx, T, Hq, d), rnd(50 + idx, T, Hkv, d), rnd(60 + idx, T, Hkv, d), rnd(70 + idx, T, Hq, d)
    scale = 0.9
    g = A.attn_bwd(q, k, v, do, spec, scale)
    dq, dk, dv = _brute.bwd(nested(q), nested(k), nested(v), nested(do), _allowed_fn(spec, Hq), scale)
    assert np.max(np.abs(g["dq"] - np.array(dq))) < 1e-11, spec.pattern
    assert np.max(np.abs(g["dk"] - np.array(dk))) < 1e-11, spec.pattern
    assert np.max(np.abs(g["dv"] - np.array(dv))) < 1e-11, spec.pattern


def test_hand_derived_causal3():
    fx = json.load(open(os.path.join(HERE, "golden", "causal3.json")))
    q, k, v, do = (np.array(fx[n]) for n in ("q", "k", "v", "do"))
    spec = M.MaskSpec(fx["pattern"], 3, 3)
    O, L = A.attn_fwd(q, k, v, spec, fx["scale"])
    assert np.max(np.abs(O - np.array(fx["o"]))) < 1e-14
    assert np.max(np.abs(L - np.array(fx["lse"]))) < 1e-14
    g = A.attn_bwd(q, k, v, do, spec, fx["scale"])
    for n in ("dq", "dk", "dv"):
        assert np.max(np.abs(g[n] - np.array(fx[n]))) < 1e-14, n


@pytest.mark.parametrize("spec", small_specs(64, seed=4), ids=lambda s: s.pattern)
def test_zero_query_closed_form(spec):
    """q = 0 makes every allowed score equal: O_i = mean of v over A_i, LSE_i = ln |A_i|."""
    T, Hq, Hkv, d = 64, 2, 1, 4
    q = np.zeros((T, Hq, d))
    k, v = rnd(1, T, Hkv, d), rnd(2, T, Hkv, d)
    O, L = A.attn_fwd(q, k, v, spec, 0.5)
    Md = M.dense(spec)
    cnt = Md.sum(axis=1)
    for i in range(T):
        if cnt[i] == 0:
            assert L[0, i] == -np.inf and np.all(O[i] == 0)
            continue
        ref = v[Md[i], 0, :].mean(axis=0)
        assert np.max(np.abs(O[i, 0] - ref)) < 1e-13
        assert abs(L[0, i] - math.log(cnt[i])) < 1e-13


def _sdpa_case(spec, T, Hq, Hkv, d, seed, scale):
    q, k, v, do = rnd(seed, T, Hq, d), rnd(seed + 1, T, Hkv, d), rnd(seed + 2, T, Hkv, d), rnd(seed + 3, T, Hq, d)
    rep = Hq // Hkv
    masks = np.stack([M.dense(spec, (h // (Hq // spec.n_groups)) if spec.n_groups > 1 else 0) for h in range(Hq)])
    empty = ~masks.any(axis=2)                                  # [Hq, T]
    masks_s = masks | empty[:, :, None]                         # keep SDPA finite on empty rows
    do = do * (~empty.T)[:, :, None]                            # those rows carry no gradient
    tq = torch.tensor(q.transpose(1, 0, 2)[None], requires_grad=True)
    tk = torch.tensor(k.transpose(1, 0, 2)[None], requires_grad=True)
    tv = torch.tensor(v.transpose(1, 0, 2)[None], requires_grad=True)
    kk = tk.repeat_interleave(rep, dim=1)
    vv = tv.repeat_interleave(rep, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, kk, vv, attn_mask=torch.tensor(masks_s[None]), scale=scale)
    o_np = o.detach().numpy()[0].transpose(1, 0, 2)
    (o * torch.tensor(do.transpose(1, 0, 2)[None])).sum().backward()
    grads = {
        "dq": tq.grad.numpy()[0].transpose(1, 0, 2),
        "dk": tk.grad.numpy()[0].transpose(1, 0, 2),
        "dv": tv.grad.numpy()[0].transpose(1, 0, 2),
    }
    return q, k, v, do, o_np, grads, empty


@pytest.mark.parametrize("spec", small_specs(96, seed=5) + [sparse_spec(96, 8, 4, 50, seed=3)],
                         ids=lambda s: s.pattern)
def test_matches_torch_sdpa_fp64(spec):
    T, Hq, Hkv, d, scale = 96, 8, 4, 16, 0.25
    q, k, v, do, o_ref, gref, empty = _sdpa_case(spec, T, Hq, Hkv, d, 11, scale)
    O, L = A.attn_fwd(q, k, v, spec, scale)
    ok = ~empty.T
    assert np.max(np.abs((O - o_ref)[ok])) < 1e-10
    g = A.attn_bwd(q, k, v, do, spec, scale)
    for n in ("dq", "dk", "dv"):
        assert np.max(np.abs(g[n] - gref[n])) < 1e-10, n


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("pattern", ["FULL", "CAUSAL", "SLIDING_WINDOW"])
def test_matches_torch_sdpa_fp64_head_dims(pattern, d):
    """The head dims the kernels are built for, at the usual scale 1/sqrt(d)."""
    T, Hq, Hkv = 48, 4, 2
    spec = [s for s in small_specs(T, seed=7) if s.pattern == pattern][0]
    scale = 1.0 / math.sqrt(d)
    q, k, v, do, o_ref, gref, empty = _sdpa_case(spec, T, Hq, Hkv, d, 21 + d, scale)
    O, L = A.attn_fwd(q, k, v, spec, scale)
    assert np.max(np.abs((O - o_ref)[~empty.T])) < 1e-10
    g = A.attn_bwd(q, k, v, do, spec, scale)
    for n in ("dq", "dk", "dv"):
        assert np.max(np.abs(g[n] - gref[n])) < 1e-10, n


@pytest.mark.parametrize("pattern", ["CAUSAL_DOCUMENT", "SHARED_QUESTION", "GLOBAL_SLIDING", "PREFIX_LM"])
def test_bwd_finite_differences(pattern):
    T, Hq, Hkv, d, scale = 12, 2, 1, 3, 0.8
    spec = [s for s in small_specs(T, seed=2) if s.pattern == pattern][0]
    q, k, v, do = rnd(1, T, Hq, d), rnd(2, T, Hkv, d), rnd(3, T, Hkv, d), rnd(4, T, Hq, d)

    def loss(q_, k_, v_):
        O, _ = A.attn_fwd(q_, k_, v_, spec, scale)
        return float(np.sum(O * do))

    g = A.attn_bwd(q, k, v, do, spec, scale)
    h = 1e-6
    for name, arr in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a0 = arr[idx]
            arr[idx] = a0 + h
            lp = loss(q, k, v)
            arr[idx] = a0 - h
            lm = loss(q, k, v)
            arr[idx] = a0
            num[idx] = (lp - lm) / (2 * h)
        err = np.linalg.norm(num - g[name]) / max(np.linalg.norm(g[name]), 1e-30)
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("spec", small_specs(80, seed=6), ids=lambda s: s.pattern)
def test_rows_sum_to_one_and_key_shift(spec):
    T, Hq, Hkv, d, scale = 80, 2, 1, 6, 0.6
    q, k = rnd(1, T, Hq, d), rnd(2, T, Hkv, d)
    ones = np.ones((T, Hkv, d))
    O, L = A.attn_fwd(q, k, ones, spec, scale)
    nonempty = np.isfinite(L[0])
    assert np.max(np.abs(O[nonempty] - 1.0)) < 1e-13
    # K -> K + 1 c^T: softmax unchanged, LSE_i shifts by scale * <q_i, c>
    v = rnd(3, T, Hkv, d)
    c = rnd(4, d)
    O1, L1 = A.attn_fwd(q, k, v, spec, scale)
    O2, L2 = A.attn_fwd(q, k + c[None, None, :], v, spec, scale)
    assert np.max(np.abs(O1 - O2)) < 1e-12
    shift = scale * np.einsum("thd,d->ht", q, c)
    fin = np.isfinite(L1)
    assert np.max(np.abs((L2 - L1 - shift)[fin]), initial=0.0) < 1e-11


def test_causal_row_equals_full_prefix():
    T, Hq, d, scale = 40, 2, 5, 0.5
    q, k, v = rnd(1, T, Hq, d), rnd(2, T, Hq, d), rnd(3, T, Hq, d)
    O, L = A.attn_fwd(q, k, v, M.MaskSpec("CAUSAL", T, T), scale)
    for i in (0, 1, 17, T - 1):
        Of, Lf = A.attn_fwd(q[i:i + 1], k[:i + 1], v[:i + 1], M.MaskSpec("FULL", 1, i + 1), scale)
        assert np.max(np.abs(O[i] - Of[0])) < 1e-13
        assert np.max(np.abs(L[:, i] - Lf[:, 0])) < 1e-13


@pytest.mark.parametrize("pattern,single", [
    ("FULL_DOCUMENT", "FULL"), ("CAUSAL_DOCUMENT", "CAUSAL"),
    ("SLIDING_WINDOW_CAUSAL_DOCUMENT", "SLIDING_WINDOW"), ("PREFIX_LM_DOCUMENT", "PREFIX_LM"),
    ("BLOCK_CAUSAL_DOCUMENT", "BLOCK_CAUSAL_DOCUMENT"),
])
def test_document_equals_concatenated_documents(pattern, single):
    T, Hq, Hkv, d, scale = 90, 4, 2, 4, 0.5
    docs = (7, 30, 1, 22, 30)
    q, k, v, do = rnd(1, T, Hq, d), rnd(2, T, Hkv, d), rnd(3, T, Hkv, d), rnd(4, T, Hq, d)
    spec = M.MaskSpec(pattern, T, T, doc_lens=docs, window=9, block=4)
    O, L = A.attn_fwd(q, k, v, spec, scale)
    g = A.attn_bwd(q, k, v, do, spec, scale)
    s0 = 0
    for Ld in docs:
        sl = slice(s0, s0 + Ld)
        sd = M.MaskSpec(single, Ld, Ld, doc_lens=(Ld,), window=9, block=4)
        Od, Ldse = A.attn_fwd(q[sl], k[sl], v[sl], sd, scale)
        gd = A.attn_bwd(q[sl], k[sl], v[sl], do[sl], sd, scale)
        assert np.max(np.abs(O[sl] - Od)) < 1e-13
        assert np.max(np.abs(L[:, sl] - Ldse)) < 1e-13
        for n in ("dq", "dk", "dv"):
            assert np.max(np.abs(g[n][sl] - gd[n])) < 1e-12
        s0 += Ld


def test_fully_masked_rows():
    """Head-tail ring step where the head half of rank 0 sees nothing: O = 0, LSE = -inf."""
    T, Hq, Hkv, d = 16, 2, 1, 4
    spec = M.MaskSpec("RING_STEP", T, T, layout="headtail", n_ranks=4, rank=0, source=2)
    q, k, v, do = rnd(1, T, Hq, d), rnd(2, T, Hkv, d), rnd(3, T, Hkv, d), rnd(4, T, Hq, d)
    O, L = A.attn_fwd(q, k, v, spec, 1.0)
    Md = M.dense(spec)
    empty = ~Md.any(axis=1)
    assert empty[:T // 2].all() and not empty[T // 2:].any()
    assert np.all(O[empty] == 0.0) and np.all(L[:, empty] == -np.inf)
    g = A.attn_bwd(q, k, v, do, spec, 1.0)
    assert np.all(g["dq"][empty] == 0.0)


def test_key_permutation_invariance_full():
    T, Hq, d = 50, 3, 7
    q, k, v = rnd(1, T, Hq, d), rnd(2, T, Hq, d), rnd(3, T, Hq, d)
    perm = np.random.default_rng(0).permutation(T)
    spec = M.MaskSpec("FULL", T, T)
    O1, L1 = A.attn_fwd(q, k, v, spec, 0.4)
    O2, L2 = A.attn_fwd(q, k[perm], v[perm], spec, 0.4)
    assert np.max(np.abs(O1 - O2)) < 1e-13 and np.max(np.abs(L1 - L2)) < 1e-13


@pytest.mark.parametrize("pattern", ["CAUSAL", "SHARED_QUESTION", "BLOCK_SPARSE"])
def test_gqa_equals_repeated_mha(pattern):
    T, Hq, Hkv, d, scale = 48, 6, 2, 4, 0.5
    rep = Hq // Hkv
    if pattern == "BLOCK_SPARSE":
        spec = sparse_spec(T, 8, Hkv, 50, seed=4)
        keep_mha = np.repeat(spec.keep, rep, axis=0)
        spec_mha = M.MaskSpec("BLOCK_SPARSE", T, T, q_edges=spec.q_edges, k_edges=spec.k_edges, keep=keep_mha)
    else:
        spec = [s for s in small_specs(T) if s.pattern == pattern][0]
        spec_mha = spec
    q, k, v, do = rnd(1, T, Hq, d), rnd(2, T, Hkv, d), rnd(3, T, Hkv, d), rnd(4, T, Hq, d)
    O, L = A.attn_fwd(q, k, v, spec, scale)
    kr, vr = np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1)
    Or, Lr = A.attn_fwd(q, kr, vr, spec_mha, scale)
    assert np.max(np.abs(O - Or)) < 1e-13 and np.max(np.abs(L - Lr)) < 1e-13
    g = A.attn_bwd(q, k, v, do, spec, scale)
    gr = A.attn_bwd(q, kr, vr, do, spec_mha, scale)
    assert np.max(np.abs(g["dq"] - gr["dq"])) < 1e-12
    for n in ("dk", "dv"):
        summed = gr[n].reshape(T, Hkv, rep, d).sum(axis=2)
        assert np.max(np.abs(g[n] - summed)) < 1e-12


@pytest.mark.parametrize("spec", small_specs(64, seed=8), ids=lambda s: s.pattern)
def test_backward_sum_invariants(spec):
    """sum_j dK_j = 0 (rows of dS sum to D_i - D_i); sum_j dV_j = sum over non-empty rows of dO."""
    T, Hq, Hkv, d, scale = 64, 4, 2, 5, 0.5
    q, k, v, do = rnd(1, T, Hq, d), rnd(2, T, Hkv, d), rnd(3, T, Hkv, d), rnd(4, T, Hq, d)
    g = A.attn_bwd(q, k, v, do, spec, scale)
    assert np.max(np.abs(g["dk"].sum(axis=0))) < 1e-12
    _, L = A.attn_fwd(q, k, v, spec, scale)
    ne = np.isfinite(L).T  # [T, Hq]
    ref = (do * ne[:, :, None]).reshape(T, Hkv, Hq // Hkv, d).sum(axis=(0, 2))
    assert np.max(np.abs(g["dv"].sum(axis=0) - ref)) < 1e-12


def test_sampled_rows_match_full():
    T, Hq, Hkv, d = 70, 4, 2, 3
    spec = small_specs(T)[4]
    q, k, v, do = rnd(1, T, Hq, d), rnd(2, T, Hkv, d), rnd(3, T, Hkv, d), rnd(4, T, Hq, d)
    rows = np.array([0, 5, 33, 69])
    O, L = A.attn_fwd(q, k, v, spec, 0.5)
    Os, Ls = A.attn_fwd(q, k, v, spec, 0.5, rows=rows)
    assert np.max(np.abs(O[rows] - Os)) < 1e-13 and np.max(np.abs(L[:, rows] - Ls)) < 1e-13
    g = A.attn_bwd(q, k, v, do, spec, 0.5)
    gs = A.attn_bwd(q, k, v, do, spec, 0.5, rows=rows, want=("dq",))
    assert np.max(np.abs(g["dq"][rows] - gs["dq"])) < 1e-13


@pytest.mark.parametrize("idx", range(N_TINY))
def test_bwd_keys_match_brute_force(idx):
    """dK / dV at chosen key columns equal the pure-Python brute force at those columns."""
    T, Hq, Hkv, d = 16, 4, 2, 3
    spec = all_tiny_specs(T)[idx]
    q, k, v, do = rnd(idx, T, Hq, d), rnd(50 + idx, T, Hkv, d), rnd(60 + idx, T, Hkv, d), rnd(70 + idx, T, Hq, d)
    keys = np.array([0, 3, 7, 8, 15])
    dk, dv = A.attn_bwd_keys(q, k, v, do, spec, 0.9, keys)
    _, bdk, bdv = _brute.bwd(nested(q), nested(k), nested(v), nested(do), _allowed_fn(spec, Hq), 0.9)
    assert np.max(np.abs(dk - np.array(bdk)[keys])) < 1e-11, spec.pattern
    assert np.max(np.abs(dv - np.array(bdv)[keys])) < 1e-11, spec.pattern


@pytest.mark.parametrize("spec", small_specs(300, seed=6), ids=lambda s: s.pattern)
def test_bwd_keys_match_full_backward(spec):
    """Across several row blocks (T = 300 > ROW_BLOCK) and for one KV head of a GQA group."""
    T, Hq, Hkv, d = 300, 4, 2, 8
    q, k, v, do = rnd(11, T, Hq, d), rnd(12, T, Hkv, d), rnd(13, T, Hkv, d), rnd(14, T, Hq, d)
    keys = np.array([0, 1, 77, 150, 255, 256, 299])
    g = A.attn_bwd(q, k, v, do, spec, 0.35)
    dk, dv = A.attn_bwd_keys(q, k, v, do, spec, 0.35, keys, kv_heads=[1])
    assert np.max(np.abs(dk[:, 0] - g["dk"][keys, 1])) < 1e-12
    assert np.max(np.abs(dv[:, 0] - g["dv"][keys, 1])) < 1e-12
    # the contributions of disjoint row sets add up to the whole
    parts = [A.attn_bwd_keys(q, k, v, do, spec, 0.35, keys, kv_heads=[1], rows=r)
             for r in (np.arange(0, 130), np.arange(130, 300))]
    assert np.max(np.abs(parts[0][0] + parts[1][0] - dk)) < 1e-12
    assert np.max(np.abs(parts[0][1] + parts[1][1] - dv)) < 1e-12
