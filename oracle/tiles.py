"""Brute-force tile classification (oracle; test infrastructure only).

For a tiling of the [Tq, Tk] mask into BM x BN tiles, each tile is
  EMPTY   (0) if no in-range element is allowed,
  FULL    (1) if every in-range element is allowed,
  PARTIAL (2) otherwise,
counting only elements with i < Tq and j < Tk (ragged edge tiles are judged
on their in-range part).  The counts come from the dense closed-form mask of
oracle.masks, row block by row block.  Visit lists: per query tile the
ascending non-EMPTY key tiles (CSR), per key tile the ascending non-EMPTY
query tiles (CSC).  The pages motivate the O(#tiles) description by the cost
of a dense O(S^2) block mask (appendix A.3 FlexAttention, A.5.2).
"""
from __future__ import annotations

import numpy as np

from . import masks as _masks

EMPTY, FULL, PARTIAL = 0, 1, 2


def tile_counts(spec, BM, BN, group=0):
    """counts [n_qt, n_kt] of allowed elements and area [n_qt, n_kt] in range."""
    Tq, Tk = spec.Tq, spec.Tk
    nqt = -(-Tq // BM)
    nkt = -(-Tk // BN)
    counts = np.zeros((nqt, nkt), dtype=np.int64)
    cols = np.arange(Tk)
    pad = nkt * BN - Tk
    for t in range(nqt):
        rows = np.arange(t * BM, min(Tq, (t + 1) * BM))
        M = _masks.allowed(spec, rows, cols, group)
        if pad:
            M = np.concatenate([M, np.zeros((M.shape[0], pad), dtype=bool)], axis=1)
        counts[t] = M.reshape(M.shape[0], nkt, BN).sum(axis=(0, 2))
    rq = np.minimum(BM, Tq - np.arange(nqt) * BM)
    rk = np.minimum(BN, Tk - np.arange(nkt) * BN)
    area = rq[:, None].astype(np.int64) * rk[None, :]
    return counts, area


def classify(spec, BM, BN, group=0):
    """Returns dict(classes uint8 [n_qt, n_kt], csr_ptr, csr_idx, csc_ptr, csc_idx, pairs)."""
    counts, area = tile_counts(spec, BM, BN, group)
    cls = np.where(counts == 0, EMPTY, np.where(counts == area, FULL, PARTIAL)).astype(np.uint8)
    nz = cls != EMPTY
    csr_ptr = np.concatenate([[0], np.cumsum(nz.sum(axis=1))]).astype(np.int64)
    csr_idx = np.concatenate([np.nonzero(nz[t])[0] for t in range(nz.shape[0])] or [np.zeros(0, np.int64)]).astype(np.int64)
    csc_ptr = np.concatenate([[0], np.cumsum(nz.sum(axis=0))]).astype(np.int64)
    csc_idx = np.concatenate([np.nonzero(nz[:, t])[0] for t in range(nz.shape[1])] or [np.zeros(0, np.int64)]).astype(np.int64)
    return {
        "classes": cls, "counts": counts, "csr_ptr": csr_ptr, "csr_idx": csr_idx,
        "csc_ptr": csc_ptr, "csc_idx": csc_idx, "pairs": int(counts.sum()),
    }
