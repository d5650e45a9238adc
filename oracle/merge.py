"""Log-sum-exp merge of partial attention results (oracle; test infrastructure only).

When the keys of one query row are split into disjoint parts t (one per ring
step of context parallelism, LongCA-bench section 2.3 and the notes' key
design 3), each part gives (O_t, LSE_t) over its own keys.  The whole-row
result is

  LSE = ln sum_t exp(LSE_t),   O = sum_t exp(LSE_t - LSE) O_t

with parts whose LSE_t = -inf weighing zero and a row with every part -inf
giving O = 0, LSE = -inf.
"""
from __future__ import annotations

import numpy as np


def merge(outs, lses):
    """outs: list of [T, H, d]; lses: list of [H, T].  Returns merged (O, LSE)."""
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lses])  # [n, H, T]
    O = np.stack([np.asarray(x, dtype=np.float64) for x in outs])  # [n, T, H, d]
    m = L.max(axis=0)
    fin = np.isfinite(m)
    msafe = np.where(fin, m, 0.0)
    w = np.where(np.isfinite(L), np.exp(L - msafe[None]), 0.0)   # [n, H, T]
    s = w.sum(axis=0)
    lse = np.where(fin, msafe + np.log(np.where(fin, s, 1.0)), -np.inf)
    wn = np.divide(w, s[None], out=np.zeros_like(w), where=fin[None])
    o = np.einsum("nht,nthd->thd", wn, O)
    return o, lse
