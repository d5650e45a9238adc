"""Host-side mask path of the library vs the oracle, bit-exact (no GPU needed).

The library's pattern -> slices generator and its mask compiler (tile
classes, per-query-tile and per-key-tile visit lists, exact pair counts) must
reproduce the oracle's brute-force classification of the closed-form mask,
at both kernel tilings, including ragged edge tiles.
"""
import numpy as np
import pytest

import mask_aware_dense_amd as mad
from _cases import small_specs
from _gpu import spec_kwargs
from mad_inputs import block_scores, doc_lengths, variable_block_sizes
from oracle import masks as M
from oracle import tiles as TL

TILINGS = {0: (128, 64), 1: (64, 128)}


def _tiling(spec, w):
    """Tile shape of tiling w: the dK/dV tiling of a block-sparse plan whose interior key-block edges
    are not all multiples of 128 (64-token blocks, variable blocks) has 64-key tiles."""
    BM, BN = TILINGS[w]
    if w == 1 and spec.k_edges is not None:
        inner = np.asarray(spec.k_edges[1:-1])
        if inner.size and not np.all(inner % 128 == 0):
            BN = 64
    return BM, BN


def _assert_plan_matches(plan, spec, group=0, which=(0, 1)):
    for w in which:
        BM, BN = _tiling(spec, w)
        info = plan.info(w)
        assert (info["BM"], info["BN"]) == (BM, BN)
        ex = plan.export(w, group)
        ref = TL.classify(spec, BM, BN, group)
        assert np.array_equal(ex["classes"], ref["classes"]), (spec.pattern, w)
        assert np.array_equal(ex["csr_ptr"], ref["csr_ptr"]) and np.array_equal(ex["csr_idx"], ref["csr_idx"])
        assert np.array_equal(ex["csc_ptr"], ref["csc_ptr"]) and np.array_equal(ex["csc_idx"], ref["csc_idx"])
        st = plan.stats(w)
        assert int(st["pairs"][group]) == ref["pairs"]
        n = ref["classes"].size
        if plan.info(w)["n_groups"] == 1:
            assert st["full"] + st["partial"] + st["empty"] == n


@pytest.mark.parametrize("T", [1, 63, 129, 1000, 2049])
@pytest.mark.parametrize("idx", range(len(M.STATIC_PATTERNS)))
def test_static_patterns_bit_exact(T, idx):
    spec = small_specs(T, seed=idx + T)[idx]
    plan = mad.mask_compile(mad.mask_slices(spec.pattern, T, **spec_kwargs(spec)), T, T)
    _assert_plan_matches(plan, spec)


@pytest.mark.parametrize("pattern", list(M.STATIC_PATTERNS))
def test_static_patterns_workload_parameters(pattern):
    """The benchmark's own parameters at 16K: window 4K (SW) / 2K (global sliding), 2K question,
    256 global tokens, blocks of 2K / 1K, documents log-uniform in [512, 16K]."""
    T = 16384
    docs = tuple(int(x) for x in doc_lengths(5, T))
    kw = dict(window=2048 if pattern == "GLOBAL_SLIDING" else 4096,
              block=2048 if pattern == "CAUSAL_BLOCKWISE" else 1024, doc_lens=docs)
    spec = M.MaskSpec(pattern, T, T, **kw)
    plan = mad.mask_compile(mad.mask_slices(pattern, T, **spec_kwargs(spec)), T, T)
    _assert_plan_matches(plan, spec, which=(0,))


@pytest.mark.parametrize("seed", range(6))
def test_random_slices_bit_exact(seed):
    """Arbitrary (possibly overlapping, windowed, non-square) slice unions."""
    rng = np.random.default_rng(seed)
    Tq, Tk = int(rng.integers(1, 700)), int(rng.integers(1, 700))
    sl = []
    for _ in range(int(rng.integers(0, 9))):
        q0, q1 = sorted(rng.integers(0, Tq + 1, size=2))
        k0, k1 = sorted(rng.integers(0, Tk + 1, size=2))
        typ = int(rng.integers(0, 2))
        win = int(rng.integers(0, 60)) if typ == 1 else 0
        sl.append((int(q0), int(q1), int(k0), int(k1), typ, win))
    arr = np.array(sl, dtype=mad.SLICE_DTYPE) if sl else np.zeros(0, dtype=mad.SLICE_DTYPE)
    plan = mad.mask_compile(arr, Tq, Tk)
    _assert_plan_matches(plan, M.MaskSpec("SLICES", Tq, Tk, slices=tuple(sl)))


@pytest.mark.parametrize("seed", range(8))
def test_varlen_slices_bit_exact(seed):
    """Batches of packed sequences (self and cross attention, empty sequences included),
    full or causal, top-left or bottom-right, with and without a window."""
    rng = np.random.default_rng(100 + seed)
    batch = int(rng.integers(1, 7))
    lq = rng.integers(0, 300, size=batch)
    lk = lq.copy() if seed % 2 == 0 else rng.integers(0, 300, size=batch)
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    for causal in (False, True):
        for br in (False, True):
            for win in (0, 37):
                if win and not causal:
                    continue
                if win and br and np.any(lk > lq):
                    with pytest.raises(mad.MadError):
                        mad.varlen_slices(cq, ck, causal=causal, window=win, bottom_right=br)
                    continue
                sl = mad.varlen_slices(cq, ck, causal=causal, window=win, bottom_right=br)
                spec = M.MaskSpec("VARLEN", int(cq[-1]), int(ck[-1]), cu_q=tuple(cq), cu_k=tuple(ck),
                                  causal=causal, bottom_right=br, varlen_window=win)
                plan = mad.mask_compile(sl, spec.Tq, spec.Tk)
                _assert_plan_matches(plan, spec)


@pytest.mark.parametrize("layout", ["contiguous", "headtail"])
def test_ring_step_slices_bit_exact(layout):
    N, C = 12, 520
    for r, s in [(0, 0), (0, 5), (11, 3), (11, 11), (4, 9), (6, 6)]:
        spec = M.MaskSpec("RING_STEP", C, C, layout=layout, n_ranks=N, rank=r, source=s)
        plan = mad.mask_compile(mad.ring_step_slices(layout, N, C, r, s), C, C)
        _assert_plan_matches(plan, spec)


@pytest.mark.parametrize("pct", [0, 20, 50, 80, 100])
def test_block_topk_bit_exact(pct):
    s = block_scores(3, 4, 37, 150)
    s[0, 0, 10:20] = 0.5  # ties
    keep = mad.block_topk(s, pct)
    ref = M.topk_keep(s, pct)
    bits = np.unpackbits(keep.view(np.uint8), axis=2, bitorder="little")[:, :, :150].astype(bool)
    assert np.array_equal(bits, ref)


def _sparse_case(T, b, G, pct, seed, variable):
    if variable:
        sizes = variable_block_sizes(seed, T)
        edges = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    else:
        edges = M.uniform_edges(T, b)
    n = len(edges) - 1
    scores = block_scores(seed, G, n, n)
    keep_bits = mad.block_topk(scores, pct)
    keep = M.topk_keep(scores, pct)
    plan = mad.sparse_plan(G, edges, edges, keep_bits)
    spec = M.MaskSpec("VARIABLE_BLOCK_SPARSE" if variable else "BLOCK_SPARSE", T, T,
                      q_edges=edges, k_edges=edges, keep=keep)
    return plan, spec


@pytest.mark.parametrize("b,variable", [(32, False), (64, False), (128, False), (100, False), (0, True)])
@pytest.mark.parametrize("pct", [20, 50, 80])
def test_sparse_plan_bit_exact(b, variable, pct):
    T, G = 2000, 3
    plan, spec = _sparse_case(T, b, G, pct, seed=pct + b, variable=variable)
    for g in range(G):
        _assert_plan_matches(plan, spec, group=g)


def test_sparse_all_kept_equals_full():
    T = 1000
    edges = M.uniform_edges(T, 64)
    n = len(edges) - 1
    keep = mad.block_topk(np.zeros((1, n, n), np.float32), 0)
    a = mad.sparse_plan(1, edges, edges, keep)
    b = mad.mask_compile(mad.mask_slices("FULL", T), T, T)
    assert np.array_equal(a.export(0)["classes"], b.export(0)["classes"])
    for w in (0, 1):  # the dK/dV tilings differ in width (64-token blocks): every tile is FULL in both
        assert np.all(a.export(w)["classes"] == 1) and np.all(b.export(w)["classes"] == 1)
    assert int(a.stats()["pairs"][0]) == T * T


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("T", [777, 4096])
def test_shared_question_sampled_answers_bit_exact(T, seed):
    """Shared Question with sampled answer lengths (some possibly empty)."""
    from mad_inputs import answer_lengths
    Q = T // 8
    lens = tuple(int(x) for x in answer_lengths(seed, T - Q, 4))
    spec = M.MaskSpec("SHARED_QUESTION", T, T, question=Q, answer_lens=lens)
    plan = mad.mask_compile(mad.mask_slices("SHARED_QUESTION", T, question=Q, answer_lens=lens), T, T)
    _assert_plan_matches(plan, spec)
    with pytest.raises(mad.MadError):
        mad.mask_slices("SHARED_QUESTION", T, question=Q, answer_lens=[1, 2])
