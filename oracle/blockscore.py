"""Block importance scores from Q and K (oracle; test infrastructure only).

LongCA-bench appendix A.3 describes the coarse stage of a block-sparse method
(VSA) as mean pooling of the QK scores over blocks, and appendix A.2 the top-k
selection of key blocks per query block with one score matrix per head (MHA)
or per KV-head group (GQA).  The score of mask group g, query block qb and key
block kb is therefore read here as the mean, over the block pair's (query,
key) positions and the group's query heads h, of the scaled dot products:

  score[g, qb, kb] = scale * mean_{i in qb, j in kb, h in g} q[i, h] . k[j, kv(h)]

A group's query heads are h = g*Hq/G .. (g+1)*Hq/G - 1 and kv(h) = h / (Hq/Hkv);
every head of a group must map to the same KV head.  The mean of the dot
products equals the dot product of the means, which is how `pooled_scores`
computes it (in fp64); `literal_scores` evaluates the definition as written,
over every (i, j, h), for small inputs only.  Top-k selection is
`masks.topk_keep`.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if hasattr(x, "float"):
        x = x.float().numpy()
    return np.asarray(x, dtype=np.float64)


def _groups(Hq, Hkv, n_groups):
    hpg = Hq // n_groups
    R = Hq // Hkv
    kv = [(g * hpg) // R for g in range(n_groups)]
    for g in range(n_groups):
        assert all(h // R == kv[g] for h in range(g * hpg, (g + 1) * hpg)), "a group spans two KV heads"
    return hpg, kv


def pooled_scores(q, k, q_edges, k_edges, n_groups: int, scale: float) -> np.ndarray:
    """[G, n_qb, n_kb] fp64 scores: scale * (block-and-group mean of Q) . (block mean of K)."""
    q, k = _f64(q), _f64(k)
    T, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    hpg, kv = _groups(Hq, Hkv, n_groups)
    qe = np.asarray(q_edges, dtype=np.int64)
    ke = np.asarray(k_edges, dtype=np.int64)
    qbar = np.stack([np.stack([q[qe[b]:qe[b + 1], g * hpg:(g + 1) * hpg].mean(axis=(0, 1))
                               for b in range(len(qe) - 1)]) for g in range(n_groups)])   # [G, nqb, d]
    kbar = np.stack([np.stack([k[ke[b]:ke[b + 1], h].mean(axis=0) for b in range(len(ke) - 1)])
                     for h in range(Hkv)])                                                 # [Hkv, nkb, d]
    return scale * np.einsum("gqd,gkd->gqk", qbar, kbar[kv])


def literal_scores(q, k, q_edges, k_edges, n_groups: int, scale: float) -> np.ndarray:
    """The definition evaluated term by term (small inputs): the mean of all scaled
    q_i . k_j over the block pair and the group's heads."""
    q, k = _f64(q), _f64(k)
    T, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    hpg, _ = _groups(Hq, Hkv, n_groups)
    R = Hq // Hkv
    nq, nk = len(q_edges) - 1, len(k_edges) - 1
    out = np.zeros((n_groups, nq, nk))
    for g in range(n_groups):
        for a in range(nq):
            for b in range(nk):
                tot, cnt = 0.0, 0
                for h in range(g * hpg, (g + 1) * hpg):
                    for i in range(q_edges[a], q_edges[a + 1]):
                        for j in range(k_edges[b], k_edges[b + 1]):
                            tot += float(np.dot(q[i, h], k[j, h // R]))
                            cnt += 1
                out[g, a, b] = scale * tot / cnt
    return out
