"""Closed-form mask predicates (oracle; test infrastructure only).

allowed(spec, rows, cols, group) returns a dense boolean block
[len(rows), len(cols)] with True where query i may attend key j.  Every
pattern is written from its definition, never from slices or tiles.

Pattern sources (LongCA-bench): 14 patterns, 12 static (6 regular, 6
heterogeneous) and 2 dynamic (section 2.1.1 "Input mask patterns"; notes' key
design 1 lists FULL, CAUSAL, sliding window, the document variants, Shared
Question, Global Sliding, Causal Blockwise, Prefix LM, Block Causal Document,
uniform and variable block-sparse).  Parameters follow the benchmark's
workload descriptions: sliding window 4K causal, Prefix LM prefix 25%, one 2K
question seen by 4 answers, 256 global tokens plus a 2K causal window, causal
blockwise blocks of 2K, Block Causal Document block 1024 (appendix A.4.1
"Block causal document").  Block-sparse: appendix A.2 (block partition,
scores, top-k per query block).

Readings where the pages are silent (the library takes the same ones):
  * sliding window W counts the key itself: i-W < j <= i
  * Prefix LM prefix P = floor(T/4), bidirectional inside the prefix
  * Shared Question answers split the rest equally, the last takes the
    remainder, unless sampled answer lengths are given (the timing runs
    sample them); the question is causal within itself
  * Global Sliding: keys 0..G-1 visible to every later query, no look-ahead
  * Causal Blockwise read literally (causal within a block, full to earlier
    blocks), which is the same set as CAUSAL
  * Block Causal Document blocks counted from each document's start
  * sixth heterogeneous mask = PREFIX_LM_DOCUMENT (prefix LM per document,
    p_d = floor(L_d/4)); parity unpinned as to identity
  * two alternative readings, kept beside the ones the workloads use:
    CAUSAL_BLOCKWISE_LAST (causal inside each block; only the last block
    also sees every earlier block, the in-context-learning layout of the
    FlashMask paper's blockwise mask) and BLOCK_CAUSAL_DOCUMENT_GLOBAL
    (block edges at multiples of B from token 0 instead of each document's
    start); parity unpinned as to which one the pages mean
  * VARLEN: a batch of packed sequences given by cumulative offsets; causal
    masks aligned top-left (key c <= row r in sequence-local offsets) or
    bottom-right (c <= r + Lk - Lq)
  * sparsity s (percent) = share of key blocks dropped per query block:
    keep k = n_kb - floor(s*n_kb/100), at least 1; ties in score broken
    toward the lower block index; one keep set per KV head (GQA shares it
    within the group, MHA has one per head)
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

STATIC_PATTERNS = (
    "FULL", "CAUSAL", "SLIDING_WINDOW", "FULL_DOCUMENT", "CAUSAL_DOCUMENT",
    "SLIDING_WINDOW_CAUSAL_DOCUMENT", "PREFIX_LM", "SHARED_QUESTION",
    "GLOBAL_SLIDING", "CAUSAL_BLOCKWISE", "BLOCK_CAUSAL_DOCUMENT",
    "PREFIX_LM_DOCUMENT", "CAUSAL_BLOCKWISE_LAST", "BLOCK_CAUSAL_DOCUMENT_GLOBAL",
)
SPARSE_PATTERNS = ("BLOCK_SPARSE", "VARIABLE_BLOCK_SPARSE")
RING_PATTERNS = ("RING_STEP",)
SLICE_PATTERNS = ("SLICES",)
VARLEN_PATTERNS = ("VARLEN",)


@dataclass
class MaskSpec:
    pattern: str
    Tq: int
    Tk: int
    window: int = 4096            # SLIDING_WINDOW*, GLOBAL_SLIDING window
    prefix: Optional[int] = None  # PREFIX_LM: default floor(T/4)
    doc_lens: tuple = ()          # document variants
    question: int = 2048          # SHARED_QUESTION
    n_answers: int = 4
    answer_lens: tuple = ()       # SHARED_QUESTION: sampled answer lengths (sum T - question) instead of equal
    global_len: int = 256         # GLOBAL_SLIDING
    block: int = 1024             # BLOCK_CAUSAL_DOCUMENT (1024), CAUSAL_BLOCKWISE (2048)
    # block-sparse: edges are cumulative boundaries (length n_blocks+1), keep is
    # bool [n_groups, n_qb, n_kb]
    q_edges: Optional[np.ndarray] = None
    k_edges: Optional[np.ndarray] = None
    keep: Optional[np.ndarray] = None
    # ring step: layout "contiguous" or "headtail", n_ranks, tokens per rank
    layout: str = "contiguous"
    n_ranks: int = 1
    rank: int = 0
    source: int = 0
    # SLICES: tuples (q0, q1, k0, k1, type 0=full 1=causal, window)
    slices: tuple = ()
    # VARLEN: cumulative offsets of the packed sequences (length batch + 1)
    cu_q: tuple = ()
    cu_k: tuple = ()
    causal: bool = True
    bottom_right: bool = False
    varlen_window: int = 0        # VARLEN causal window (0: none)

    @property
    def n_groups(self) -> int:
        return 1 if self.keep is None else int(self.keep.shape[0])


def _doc_index(doc_lens, pos):
    """Document id and document start for each position in `pos`."""
    ends = np.cumsum(np.asarray(doc_lens, dtype=np.int64))
    starts = ends - np.asarray(doc_lens, dtype=np.int64)
    d = np.searchsorted(ends, pos, side="right")
    return d, starts[d], np.asarray(doc_lens, dtype=np.int64)[d]


def _answer_segment(T, question, n_answers, pos, answer_lens=()):
    """Segment id: 0 for the question, 1..n for answers (equal split of the rest, or the given
    answer lengths, which sum to T - question)."""
    if len(answer_lens):
        ends = question + np.cumsum(np.asarray(answer_lens, dtype=np.int64))
        return np.where(pos < question, 0, np.searchsorted(ends, pos, side="right") + 1)
    rest = T - question
    base = rest // n_answers
    a = pos - question
    if base > 0:
        ans = np.minimum(a // base, n_answers - 1) + 1
    else:  # fewer answer tokens than answers: the first n-1 answers are empty
        ans = np.full_like(pos, n_answers)
    return np.where(pos < question, 0, ans)


def topk_keep(scores: np.ndarray, sparsity_pct: int) -> np.ndarray:
    """Top-k key blocks per (group, query block) from block scores.

    Appendix A.2: per query block the top-k key blocks by score are kept; the
    sparsity ratio converts directly to k.  k = n_kb - floor(pct*n_kb/100),
    at least 1.  Ordering: higher score first, equal scores by lower index.
    """
    G, nq, nk = scores.shape
    k = max(1, nk - (int(sparsity_pct) * nk) // 100)
    order = np.argsort(-scores.astype(np.float64), axis=2, kind="stable")
    keep = np.zeros(scores.shape, dtype=bool)
    np.put_along_axis(keep, order[:, :, :k], True, axis=2)
    return keep


def uniform_edges(T: int, b: int) -> np.ndarray:
    """Block boundaries 0, b, 2b, ..., T (the last block may be short)."""
    e = list(range(0, T, b)) + [T]
    return np.asarray(e, dtype=np.int64)


def _ring_positions(spec: MaskSpec, local, which: str):
    """Global sequence position of local token indices on a ring rank.

    contiguous: rank r holds tokens [r*C, (r+1)*C).  headtail: the sequence is
    cut into 2N halves of C/2 and rank r holds halves r and 2N-1-r, which
    balances causal work across ranks (notes' key design 3: dual-chunk
    head-tail reordering).
    """
    r = spec.rank if which == "q" else spec.source
    C = spec.Tq if which == "q" else spec.Tk
    if spec.layout == "contiguous":
        return r * C + local
    half = C // 2
    a, b = r, 2 * spec.n_ranks - 1 - r
    return np.where(local < half, a * half + local, b * half + (local - half))


def allowed(spec: MaskSpec, rows, cols, group: int = 0) -> np.ndarray:
    """Dense boolean mask block for query indices `rows` and key indices `cols`."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    p = spec.pattern
    T = spec.Tq
    if p == "FULL":
        return np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if p == "CAUSAL":
        return j <= i
    if p == "SLIDING_WINDOW":
        W = spec.window
        return (j <= i) & (j > i - W)
    if p in ("FULL_DOCUMENT", "CAUSAL_DOCUMENT", "SLIDING_WINDOW_CAUSAL_DOCUMENT",
             "BLOCK_CAUSAL_DOCUMENT", "PREFIX_LM_DOCUMENT", "BLOCK_CAUSAL_DOCUMENT_GLOBAL"):
        di, si, Li = _doc_index(spec.doc_lens, i)
        dj, _, _ = _doc_index(spec.doc_lens, j)
        same = di == dj
        if p == "FULL_DOCUMENT":
            return same
        if p == "CAUSAL_DOCUMENT":
            return same & (j <= i)
        if p == "SLIDING_WINDOW_CAUSAL_DOCUMENT":
            W = spec.window
            return same & (j <= i) & (j > i - W)
        if p == "BLOCK_CAUSAL_DOCUMENT":
            B = spec.block
            return same & (((j - si) // B) <= ((i - si) // B))
        if p == "BLOCK_CAUSAL_DOCUMENT_GLOBAL":
            B = spec.block
            return same & ((j // B) <= (i // B))
        # PREFIX_LM_DOCUMENT
        pd = Li // 4
        return same & ((j - si) <= np.maximum(i - si, pd - 1))
    if p == "PREFIX_LM":
        P = (T // 4) if spec.prefix is None else spec.prefix
        return j <= np.maximum(i, P - 1)
    if p == "SHARED_QUESTION":
        Q = spec.question
        si = _answer_segment(T, Q, spec.n_answers, i, spec.answer_lens)
        sj = _answer_segment(T, Q, spec.n_answers, j, spec.answer_lens)
        return (j <= i) & ((j < Q) | (si == sj))
    if p == "GLOBAL_SLIDING":
        G, W = spec.global_len, spec.window
        return (j <= i) & ((j < G) | (i - j < W))
    if p == "CAUSAL_BLOCKWISE":
        B = spec.block
        bi, bj = i // B, j // B
        return (bj < bi) | ((bj == bi) & (j <= i))
    if p == "CAUSAL_BLOCKWISE_LAST":
        B = spec.block
        bi, bj = i // B, j // B
        last = (T - 1) // B
        return ((bj == bi) & (j <= i)) | ((bi == last) & (bj < bi))
    if p == "VARLEN":
        cq = np.asarray(spec.cu_q, dtype=np.int64)
        ck = np.asarray(spec.cu_k if spec.cu_k else spec.cu_q, dtype=np.int64)
        # sequence of each token; tokens past the last offset belong to none
        bi = np.searchsorted(cq, i, side="right") - 1
        bj = np.searchsorted(ck, j, side="right") - 1
        nb = len(cq) - 1
        ok = (bi >= 0) & (bi < nb) & (bj >= 0) & (bj < nb) & (bi == bj)
        bic = np.clip(bi, 0, max(nb - 1, 0))
        bjc = np.clip(bj, 0, max(nb - 1, 0))
        if not spec.causal or nb == 0:
            return ok
        r = i - cq[bic]
        c = j - ck[bjc]
        shift = (ck[bic + 1] - ck[bic]) - (cq[bic + 1] - cq[bic]) if spec.bottom_right else 0
        m = ok & (c <= r + shift)
        if spec.varlen_window > 0:
            m &= (r + shift - c) < spec.varlen_window
        return m
    if p in ("BLOCK_SPARSE", "VARIABLE_BLOCK_SPARSE"):
        qb = np.searchsorted(spec.q_edges, i, side="right") - 1
        kb = np.searchsorted(spec.k_edges, j, side="right") - 1
        return spec.keep[group][qb, kb]
    if p == "RING_STEP":
        gi = _ring_positions(spec, i, "q")
        gj = _ring_positions(spec, j, "k")
        return gi >= gj
    if p == "SLICES":
        # the unified mask format itself: union of (q_range, k_range, full |
        # causal[, window]) slices, causal aligned at each slice's top-left
        out = np.zeros((i.shape[0], j.shape[1]), dtype=bool)
        for (q0, q1, k0, k1, typ, win) in spec.slices:
            m = (i >= q0) & (i < q1) & (j >= k0) & (j < k1)
            if typ == 1:
                m = m & ((j - k0) <= (i - q0))
                if win > 0:
                    m = m & ((i - q0) - (j - k0) < win)
            out |= m
        return out
    raise ValueError(f"unknown mask pattern {p!r}")


def dense(spec: MaskSpec, group: int = 0) -> np.ndarray:
    """Whole [Tq, Tk] mask (small sizes only)."""
    return allowed(spec, np.arange(spec.Tq), np.arange(spec.Tk), group)


def pair_count(spec: MaskSpec, group: int = 0, row_block: int = 1024) -> int:
    """Exact number of allowed (i, j) pairs, counted row block by row block."""
    n = 0
    cols = np.arange(spec.Tk)
    for r0 in range(0, spec.Tq, row_block):
        rows = np.arange(r0, min(spec.Tq, r0 + row_block))
        n += int(np.count_nonzero(allowed(spec, rows, cols, group)))
    return n
