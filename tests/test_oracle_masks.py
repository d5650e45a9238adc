"""Pins for the oracle's mask predicates, tile classifier, top-k and merge."""
import numpy as np
import pytest

from _cases import small_specs, sparse_spec
from mad_inputs import block_scores, doc_lengths, variable_block_sizes
from oracle import attention as A
from oracle import masks as M
from oracle import merge as MG
from oracle import tiles as TL


# ---- closed-form pair counts (sums written out from each definition) ----

def sw_pairs(T, W):
    return sum(min(i + 1, W) for i in range(T))


def plm_pairs(T, P):
    return sum(max(i, P - 1) + 1 for i in range(T))


def sq_pairs(T, Q, n):
    rest = T - Q
    base = rest // n
    lens = [base] * (n - 1) + [rest - base * (n - 1)]
    return Q * (Q + 1) // 2 + sum(L * Q + L * (L + 1) // 2 for L in lens)


def gs_pairs(T, G, W):
    return sum(min(i + 1, W) + max(0, min(G, i - W + 1)) for i in range(T))


@pytest.mark.parametrize("T", [1000, 4096])
def test_pair_counts_closed_form(T):
    assert M.pair_count(M.MaskSpec("FULL", T, T)) == T * T
    assert M.pair_count(M.MaskSpec("CAUSAL", T, T)) == T * (T + 1) // 2
    W = T // 8
    assert M.pair_count(M.MaskSpec("SLIDING_WINDOW", T, T, window=W)) == sw_pairs(T, W)
    assert M.pair_count(M.MaskSpec("PREFIX_LM", T, T)) == plm_pairs(T, T // 4)
    assert M.pair_count(M.MaskSpec("SHARED_QUESTION", T, T, question=T // 16, n_answers=4)) == sq_pairs(T, T // 16, 4)
    assert M.pair_count(M.MaskSpec("GLOBAL_SLIDING", T, T, global_len=T // 128, window=T // 16)) == gs_pairs(T, T // 128, T // 16)
    assert M.pair_count(M.MaskSpec("CAUSAL_BLOCKWISE", T, T, block=T // 16)) == T * (T + 1) // 2


@pytest.mark.slow
def test_pair_counts_32k_workload():
    """The 32K heterogeneous workload: 4K window, 25% prefix, 2K question + 4 answers, 256 global + 2K window."""
    T = 32768
    assert sw_pairs(T, 4096) == 125_831_168
    assert M.pair_count(M.MaskSpec("SLIDING_WINDOW", T, T, window=4096)) == 125_831_168
    assert M.pair_count(M.MaskSpec("PREFIX_LM", T, T)) == plm_pairs(T, 8192) == 570_437_632
    assert M.pair_count(M.MaskSpec("SHARED_QUESTION", T, T)) == sq_pairs(T, 2048, 4) == 182_992_896
    assert M.pair_count(M.MaskSpec("GLOBAL_SLIDING", T, T, window=2048)) == gs_pairs(T, 256, 2048) == 72_844_416


def test_document_pair_counts():
    docs = tuple(int(x) for x in doc_lengths(3, 20000))
    T = sum(docs)
    assert T == 20000
    assert M.pair_count(M.MaskSpec("FULL_DOCUMENT", T, T, doc_lens=docs)) == sum(L * L for L in docs)
    assert M.pair_count(M.MaskSpec("CAUSAL_DOCUMENT", T, T, doc_lens=docs)) == sum(L * (L + 1) // 2 for L in docs)
    W = 700
    assert M.pair_count(M.MaskSpec("SLIDING_WINDOW_CAUSAL_DOCUMENT", T, T, doc_lens=docs, window=W)) == \
        sum(sw_pairs(L, W) for L in docs)
    assert M.pair_count(M.MaskSpec("PREFIX_LM_DOCUMENT", T, T, doc_lens=docs)) == sum(plm_pairs(L, L // 4) for L in docs)
    B = 300
    bcd = 0
    for L in docs:  # block b (from the document start) sees blocks 0..b in full
        for i in range(L):
            bcd += min(L, (i // B + 1) * B)
    assert M.pair_count(M.MaskSpec("BLOCK_CAUSAL_DOCUMENT", T, T, doc_lens=docs, block=B)) == bcd


def _eq(a, b):
    return np.array_equal(M.dense(a), M.dense(b))


def test_special_case_reductions():
    T = 97
    docs = (10, 40, 1, 46)
    C = M.MaskSpec("CAUSAL", T, T)
    assert _eq(M.MaskSpec("SLIDING_WINDOW", T, T, window=T), C)
    assert _eq(M.MaskSpec("SLIDING_WINDOW", T, T, window=5 * T), C)
    assert _eq(M.MaskSpec("PREFIX_LM", T, T, prefix=1), C)
    assert _eq(M.MaskSpec("PREFIX_LM", T, T, prefix=0), C)
    for B in (1, 2, 7, 50, 200):
        assert _eq(M.MaskSpec("CAUSAL_BLOCKWISE", T, T, block=B), C)
    assert _eq(M.MaskSpec("BLOCK_CAUSAL_DOCUMENT", T, T, doc_lens=docs, block=1),
               M.MaskSpec("CAUSAL_DOCUMENT", T, T, doc_lens=docs))
    assert _eq(M.MaskSpec("BLOCK_CAUSAL_DOCUMENT", T, T, doc_lens=docs, block=46),
               M.MaskSpec("FULL_DOCUMENT", T, T, doc_lens=docs))
    assert _eq(M.MaskSpec("SHARED_QUESTION", T, T, question=30, n_answers=1), C)
    assert _eq(M.MaskSpec("GLOBAL_SLIDING", T, T, global_len=0, window=9),
               M.MaskSpec("SLIDING_WINDOW", T, T, window=9))
    one = (T,)
    assert _eq(M.MaskSpec("FULL_DOCUMENT", T, T, doc_lens=one), M.MaskSpec("FULL", T, T))
    assert _eq(M.MaskSpec("CAUSAL_DOCUMENT", T, T, doc_lens=one), C)
    assert _eq(M.MaskSpec("SLIDING_WINDOW_CAUSAL_DOCUMENT", T, T, doc_lens=one, window=11),
               M.MaskSpec("SLIDING_WINDOW", T, T, window=11))
    assert _eq(M.MaskSpec("PREFIX_LM_DOCUMENT", T, T, doc_lens=one), M.MaskSpec("PREFIX_LM", T, T))
    # block-sparse: everything kept is FULL; only the diagonal kept is block-diagonal
    sizes = variable_block_sizes(1, T, lo=3, hi=20)
    edges = np.concatenate([[0], np.cumsum(sizes)])
    n = len(sizes)
    allk = M.MaskSpec("VARIABLE_BLOCK_SPARSE", T, T, q_edges=edges, k_edges=edges, keep=np.ones((1, n, n), bool))
    assert _eq(allk, M.MaskSpec("FULL", T, T))
    diag = M.MaskSpec("VARIABLE_BLOCK_SPARSE", T, T, q_edges=edges, k_edges=edges, keep=np.eye(n, dtype=bool)[None])
    assert _eq(diag, M.MaskSpec("FULL_DOCUMENT", T, T, doc_lens=tuple(int(x) for x in sizes)))
    keep0 = M.topk_keep(block_scores(0, 1, n, n), 0)
    assert keep0.all()


def test_topk_keep():
    s = block_scores(7, 3, 5, 40)
    for pct in (20, 50, 80):
        keep = M.topk_keep(s, pct)
        k = 40 - (pct * 40) // 100
        assert (keep.sum(axis=2) == k).all()
        for g in range(3):
            for r in range(5):
                assert s[g, r][keep[g, r]].min() >= s[g, r][~keep[g, r]].max()
    # ties go to the lower index
    tie = np.zeros((1, 1, 6), np.float32)
    tie[0, 0, [1, 3, 4]] = 1.0
    keep = M.topk_keep(tie, 50)  # k = 3
    assert keep[0, 0].tolist() == [False, True, False, True, True, False]
    keep = M.topk_keep(tie, 80)  # k = 6 - 4 = 2
    assert keep[0, 0].tolist() == [False, True, False, True, False, False]
    assert M.topk_keep(tie, 100)[0, 0].sum() == 1  # at least one block


def test_generators_cover_total():
    for T in (1, 511, 8192, 49152):
        dl = doc_lengths(0, T)
        assert dl.sum() == T and dl.min() >= 1 and dl.max() <= 16384
        vs = variable_block_sizes(0, T)
        assert vs.sum() == T and vs.min() >= 1 and vs.max() <= 256


@pytest.mark.parametrize("layout", ["contiguous", "headtail"])
def test_ring_steps_tile_causal_exactly_once(layout):
    N, C = 3, 8
    T = N * C
    cover = np.zeros((T, T), dtype=np.int64)
    for r in range(N):
        for s in range(N):
            spec = M.MaskSpec("RING_STEP", C, C, layout=layout, n_ranks=N, rank=r, source=s)
            Md = M.dense(spec)
            gq = M._ring_positions(spec, np.arange(C), "q")
            gk = M._ring_positions(spec, np.arange(C), "k")
            for i in range(C):
                for j in range(C):
                    if Md[i, j]:
                        cover[gq[i], gk[j]] += 1
    assert np.array_equal(cover, np.tril(np.ones((T, T), dtype=np.int64)))


# ---- tile classifier ----

def _brute_tiles(spec, BM, BN, group=0):
    Md = M.dense(spec, group)
    nqt, nkt = -(-spec.Tq // BM), -(-spec.Tk // BN)
    cls = np.zeros((nqt, nkt), np.uint8)
    cnt = np.zeros((nqt, nkt), np.int64)
    for a in range(nqt):
        for b in range(nkt):
            blk = Md[a * BM:(a + 1) * BM, b * BN:(b + 1) * BN]
            c = int(blk.sum())
            cnt[a, b] = c
            cls[a, b] = 0 if c == 0 else (1 if c == blk.size else 2)
    return cls, cnt


@pytest.mark.parametrize("BM,BN", [(8, 4), (16, 16), (5, 7)])
def test_classifier_matches_per_tile_brute_force(BM, BN):
    T = 61
    specs = small_specs(T, seed=9) + [sparse_spec(T, 6, 2, 50, seed=2)]
    for spec in specs:
        for g in range(spec.n_groups):
            r = TL.classify(spec, BM, BN, g)
            cls, cnt = _brute_tiles(spec, BM, BN, g)
            assert np.array_equal(r["classes"], cls), spec.pattern
            assert np.array_equal(r["counts"], cnt), spec.pattern
            assert r["pairs"] == M.pair_count(spec, g)
            for t in range(cls.shape[0]):
                lst = r["csr_idx"][r["csr_ptr"][t]:r["csr_ptr"][t + 1]]
                assert lst.tolist() == [b for b in range(cls.shape[1]) if cls[t, b] != 0]
            for b in range(cls.shape[1]):
                lst = r["csc_idx"][r["csc_ptr"][b]:r["csc_ptr"][b + 1]]
                assert lst.tolist() == [t for t in range(cls.shape[0]) if cls[t, b] != 0]


def test_classifier_shapes_of_regular_masks():
    T, B = 64, 8
    r = TL.classify(M.MaskSpec("FULL", T, T), B, B)
    assert (r["classes"] == TL.FULL).all()
    r = TL.classify(M.MaskSpec("CAUSAL", T, T), B, B)
    n = T // B
    exp = np.where(np.tri(n, n, -1, dtype=bool), TL.FULL, TL.EMPTY)
    np.fill_diagonal(exp, TL.PARTIAL)
    assert np.array_equal(r["classes"], exp)


# ---- merge ----

def test_merge_of_key_partition_equals_whole():
    T, Hq, d = 30, 2, 4
    rng = np.random.default_rng(0)
    q, k, v = rng.standard_normal((T, Hq, d)), rng.standard_normal((T, Hq, d)), rng.standard_normal((T, Hq, d))
    O, L = A.attn_fwd(q, k, v, M.MaskSpec("FULL", T, T), 0.5)
    parts = [slice(0, 7), slice(7, 8), slice(8, 30)]
    outs, lses = [], []
    for p in parts:
        n = p.stop - p.start
        o, l = A.attn_fwd(q, k[p], v[p], M.MaskSpec("FULL", T, n), 0.5)
        outs.append(o)
        lses.append(l)
    Om, Lm = MG.merge(outs, lses)
    assert np.max(np.abs(Om - O)) < 1e-13 and np.max(np.abs(Lm - L)) < 1e-13


@pytest.mark.parametrize("layout", ["contiguous", "headtail"])
def test_ring_merge_equals_dense_causal(layout):
    N, C, Hq, Hkv, d = 4, 12, 2, 1, 3
    T = N * C
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((T, Hq, d)), rng.standard_normal((T, Hkv, d)), rng.standard_normal((T, Hkv, d))
    Oall, Lall = A.attn_fwd(q, k, v, M.MaskSpec("CAUSAL", T, T), 0.7)
    for r in range(N):
        spec_r = M.MaskSpec("RING_STEP", C, C, layout=layout, n_ranks=N, rank=r, source=0)
        gq = M._ring_positions(spec_r, np.arange(C), "q")
        outs, lses = [], []
        for s in range(N):
            spec = M.MaskSpec("RING_STEP", C, C, layout=layout, n_ranks=N, rank=r, source=s)
            gk = M._ring_positions(spec, np.arange(C), "k")
            o, l = A.attn_fwd(q[gq], k[gk], v[gk], spec, 0.7)
            outs.append(o)
            lses.append(l)
        Om, Lm = MG.merge(outs, lses)
        assert np.max(np.abs(Om - Oall[gq])) < 1e-13
        assert np.max(np.abs(Lm - Lall[:, gq])) < 1e-13


def test_slice_union_matches_closed_forms():
    """Hand-written slice lists (the unified format) rasterise to the closed-form masks."""
    T = 50
    P = T // 4
    cases = [
        ("CAUSAL", [(0, T, 0, T, 1, 0)], {}),
        ("SLIDING_WINDOW", [(0, T, 0, T, 1, 7)], dict(window=7)),
        ("PREFIX_LM", [(0, T, 0, P, 0, 0), (P, T, P, T, 1, 0)], {}),
        ("GLOBAL_SLIDING", [(0, T, 0, T, 1, 9), (9, T, 0, 4, 1, 0)], dict(global_len=4, window=9)),
        ("FULL_DOCUMENT", [(0, 20, 0, 20, 0, 0), (20, 50, 20, 50, 0, 0)], dict(doc_lens=(20, 30))),
    ]
    for pat, sl, kw in cases:
        a = M.dense(M.MaskSpec("SLICES", T, T, slices=tuple(sl)))
        b = M.dense(M.MaskSpec(pat, T, T, **kw))
        assert np.array_equal(a, b), pat
    # overlapping slices: the union counts each pair once
    a = M.dense(M.MaskSpec("SLICES", T, T, slices=((0, T, 0, T, 1, 0), (0, T, 0, T, 1, 0), (5, 9, 0, 40, 0, 0))))
    ref = np.tri(T, T, dtype=bool)
    ref[5:9, 0:40] = True
    assert np.array_equal(a, ref)


# ---- alternative readings and the varlen layout: special cases and closed forms ----

def _blocks(T, B):
    return [min(B, T - b0) for b0 in range(0, T, B)]


@pytest.mark.parametrize("T,B", [(1000, 333), (1000, 1), (1000, 1000), (1000, 4000), (77, 10), (64, 32)])
def test_causal_blockwise_last(T, B):
    """Causal inside each block; the last block also sees all earlier blocks.

    Pair count: every block its own triangle, plus the last block's rows times
    all earlier keys.  B >= T is CAUSAL; two blocks are CAUSAL too (the last
    block then sees everything before it); B = 1 is the diagonal plus a full
    last row (2T - 1 pairs)."""
    spec = M.MaskSpec("CAUSAL_BLOCKWISE_LAST", T, T, block=B)
    L = _blocks(T, B)
    want = sum(x * (x + 1) // 2 for x in L) + L[-1] * (T - L[-1])
    assert M.pair_count(spec) == want
    rows = np.arange(T)
    m = M.allowed(spec, rows, rows)
    if len(L) <= 2:
        assert np.array_equal(m, M.allowed(M.MaskSpec("CAUSAL", T, T), rows, rows))
    if B == 1:
        assert want == 2 * T - 1
    # rows outside the last block never look outside their own block
    bi = rows // B
    assert not np.any(m & (bi[:, None] != bi[None, :]) & (bi[:, None] != bi[-1]))


def test_block_causal_document_global():
    """Block edges at multiples of B from token 0.

    B >= T gives FULL_DOCUMENT, B = 1 gives CAUSAL_DOCUMENT, and documents
    that start on multiples of B give the per-document reading."""
    T = 1000
    docs = tuple(int(x) for x in doc_lengths(11, T, lo=20, hi=400))
    rows = np.arange(T)

    def m(p, **kw):
        return M.allowed(M.MaskSpec(p, T, T, doc_lens=docs, **kw), rows, rows)

    assert np.array_equal(m("BLOCK_CAUSAL_DOCUMENT_GLOBAL", block=T), m("FULL_DOCUMENT"))
    assert np.array_equal(m("BLOCK_CAUSAL_DOCUMENT_GLOBAL", block=1), m("CAUSAL_DOCUMENT"))
    aligned = (200, 100, 300, 400)
    mg = M.allowed(M.MaskSpec("BLOCK_CAUSAL_DOCUMENT_GLOBAL", T, T, doc_lens=aligned, block=100), rows, rows)
    md = M.allowed(M.MaskSpec("BLOCK_CAUSAL_DOCUMENT", T, T, doc_lens=aligned, block=100), rows, rows)
    assert np.array_equal(mg, md)
    # a document [s, e) contributes, per global block g it meets, (rows in the block) x (keys s .. block end)
    B = 64
    want, s0 = 0, 0
    for L in docs:
        e = s0 + L
        for g0 in range(s0 // B * B, e, B):
            r0, r1 = max(s0, g0), min(e, g0 + B)
            want += (r1 - r0) * (r1 - s0)
        s0 = e
    assert M.pair_count(M.MaskSpec("BLOCK_CAUSAL_DOCUMENT_GLOBAL", T, T, doc_lens=docs, block=B)) == want


def test_varlen_reduces_to_document_patterns():
    """With cu_k = cu_q, VARLEN is the document family: FULL_DOCUMENT, CAUSAL_DOCUMENT
    (either alignment) and SLIDING_WINDOW_CAUSAL_DOCUMENT; one sequence is FULL / CAUSAL."""
    docs = tuple(int(x) for x in doc_lengths(12, 900, lo=10, hi=300))
    T = sum(docs)
    cu = tuple(int(x) for x in np.concatenate([[0], np.cumsum(docs)]))
    rows = np.arange(T)

    def v(**kw):
        return M.allowed(M.MaskSpec("VARLEN", T, T, cu_q=cu, **kw), rows, rows)

    def d(p, **kw):
        return M.allowed(M.MaskSpec(p, T, T, doc_lens=docs, **kw), rows, rows)

    assert np.array_equal(v(causal=False), d("FULL_DOCUMENT"))
    assert np.array_equal(v(causal=True), d("CAUSAL_DOCUMENT"))
    assert np.array_equal(v(causal=True, bottom_right=True), d("CAUSAL_DOCUMENT"))
    assert np.array_equal(v(causal=True, varlen_window=50), d("SLIDING_WINDOW_CAUSAL_DOCUMENT", window=50))
    one = M.MaskSpec("VARLEN", T, T, cu_q=(0, T), causal=True)
    assert np.array_equal(M.allowed(one, rows, rows), M.allowed(M.MaskSpec("CAUSAL", T, T), rows, rows))


@pytest.mark.parametrize("lq,lk", [(100, 250), (250, 100), (7, 7), (0, 5), (5, 0)])
def test_varlen_cross_attention_counts(lq, lk):
    """Cross attention (Lq != Lk) in one sequence of a batch: top-left row r sees keys 0..r,
    bottom-right row r sees keys 0..r + Lk - Lq (both clipped to [0, Lk))."""
    pre_q, pre_k = 30, 40  # a first sequence before it
    cq, ck = (0, pre_q, pre_q + lq), (0, pre_k, pre_k + lk)
    for br in (False, True):
        spec = M.MaskSpec("VARLEN", cq[-1], ck[-1], cu_q=cq, cu_k=ck, causal=True, bottom_right=br)
        sh = lk - lq if br else 0
        seq2 = sum(min(lk, max(0, r + 1 + sh)) for r in range(lq))
        seq1 = sum(min(pre_k, max(0, r + 1 + ((pre_k - pre_q) if br else 0))) for r in range(pre_q))
        assert M.pair_count(spec) == seq1 + seq2


def sq_pairs_lens(Q, lens):
    return Q * (Q + 1) // 2 + sum(L * Q + L * (L + 1) // 2 for L in lens)


@pytest.mark.parametrize("seed", range(4))
def test_shared_question_sampled_answers(seed):
    """Sampled answer lengths (the timing runs' Shared Question samples): the pair count follows
    from the lengths; lengths equal to the equal split give the default mask; a single answer of
    the whole rest gives CAUSAL."""
    from mad_inputs import answer_lengths
    T, Q = 3000, 512
    lens = tuple(int(x) for x in answer_lengths(seed, T - Q, 4))
    assert sum(lens) == T - Q and len(lens) == 4 and min(lens) >= 0
    spec = M.MaskSpec("SHARED_QUESTION", T, T, question=Q, answer_lens=lens)
    assert M.pair_count(spec) == sq_pairs_lens(Q, lens)
    base = (T - Q) // 4
    eq = (base, base, base, T - Q - 3 * base)
    assert np.array_equal(M.dense(M.MaskSpec("SHARED_QUESTION", T, T, question=Q, answer_lens=eq)),
                          M.dense(M.MaskSpec("SHARED_QUESTION", T, T, question=Q, n_answers=4)))
    assert np.array_equal(M.dense(M.MaskSpec("SHARED_QUESTION", T, T, question=Q, answer_lens=(T - Q,))),
                          M.dense(M.MaskSpec("CAUSAL", T, T)))
    # an empty answer changes nothing for the others
    z = (lens[0], 0, lens[1] + lens[2], lens[3])
    assert M.pair_count(M.MaskSpec("SHARED_QUESTION", T, T, question=Q, answer_lens=z)) == sq_pairs_lens(Q, z)
