"""Softmax attention forward and backward in fp64 (oracle; test infrastructure only).

Definition (standard quadratic softmax attention, LongCA-bench section 1 and
the naive step-by-step baseline of section 3.1): for query head h with KV head
g = floor(h / (Hq/Hkv)) and query row i with allowed key set A_i,

  S_ij   = scale * <q_i, k_j>
  m_i    = max_{j in A_i} S_ij,   l_i = sum_{j in A_i} exp(S_ij - m_i)
  P_ij   = exp(S_ij - m_i) / l_i on A_i, 0 elsewhere
  O_i    = sum_j P_ij v_j,        LSE_i = m_i + ln l_i
  A_i empty:  O_i = 0, LSE_i = -inf

Backward, for a given O and LSE (the oracle's own, or merged ones):
  P_ij  = exp(S_ij - LSE_i) on A_i (0 if LSE_i = -inf)
  D_i   = <dO_i, O_i>
  dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - D_i)
  dQ_i  = scale * sum_j dS_ij k_j
  dK_j  = scale * sum_{h in group} sum_i dS^h_ij q^h_i
  dV_j  = sum_{h in group} sum_i P^h_ij dO^h_i

Arrays are numpy, layout [T, H, d].  The mask comes from oracle.masks.allowed
only.  Rows are processed in blocks; key columns whose mask column is all
False inside a row block are dropped before the matmul (the oracle decides
emptiness itself from the dense mask block).  Nothing else is blocked, fused
or reordered.
"""
from __future__ import annotations

import numpy as np

from . import masks as _masks

ROW_BLOCK = 256


def to_f64(x) -> np.ndarray:
    """bf16/fp32 torch tensor or numpy array -> fp64 numpy (exact upcast)."""
    if hasattr(x, "detach"):
        return x.detach().to("cpu").float().numpy().astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def _head_group(h, Hq, Hkv):
    return h // (Hq // Hkv)


def _mask_group(spec, h, Hq):
    G = spec.n_groups
    return h // (Hq // G) if G > 1 else 0


def fwd_rows(q, k, v, spec, scale, h, rows):
    """O [len(rows), d] and LSE [len(rows)] for query head h and the given rows."""
    Hq, Hkv = q.shape[1], k.shape[1]
    g = _head_group(h, Hq, Hkv)
    mg = _mask_group(spec, h, Hq)
    M = _masks.allowed(spec, rows, np.arange(k.shape[0]), mg)
    cols = np.nonzero(M.any(axis=0))[0]
    d = v.shape[2]
    O = np.zeros((len(rows), d))
    L = np.full(len(rows), -np.inf)
    if cols.size == 0:
        return O, L
    Mc = M[:, cols]
    S = scale * (q[rows, h, :] @ k[cols, g, :].T)
    S = np.where(Mc, S, -np.inf)
    has = Mc.any(axis=1)
    m = np.where(has, S.max(axis=1, initial=-np.inf), 0.0)
    E = np.where(Mc, np.exp(S - m[:, None]), 0.0)
    l = E.sum(axis=1)
    P = np.divide(E, l[:, None], out=np.zeros_like(E), where=has[:, None])
    O = P @ v[cols, g, :]
    L = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return O, L


def attn_fwd(q, k, v, spec, scale, heads=None, rows=None):
    """Forward pass.  Returns O [Tq, Hq, d] (or [len(rows), Hq, d]) and LSE [Hq, Tq]."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    Tq, Hq, d = q.shape
    rows_all = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = range(Hq) if heads is None else heads
    O = np.zeros((len(rows_all), Hq, d))
    L = np.full((Hq, len(rows_all)), -np.inf)
    for h in heads:
        for r0 in range(0, len(rows_all), ROW_BLOCK):
            rr = rows_all[r0:r0 + ROW_BLOCK]
            o, l = fwd_rows(q, k, v, spec, scale, h, rr)
            O[r0:r0 + len(rr), h, :] = o
            L[h, r0:r0 + len(rr)] = l
    return O, L


def attn_bwd(q, k, v, do, spec, scale, o=None, lse=None, heads=None,
             rows=None, want=("dq", "dk", "dv")):
    """Backward pass.  Returns dict with dq [rows, Hq, d], dk, dv [Tk, Hkv, d].

    If o / lse are not given, the oracle's own fp64 forward supplies them.
    `rows` restricts the query rows (dK/dV then hold only those rows'
    contributions); `heads` restricts the query heads.
    """
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    Tq, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    rows_all = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    dq = np.zeros((len(rows_all), Hq, d))
    dk = np.zeros((Tk, Hkv, d))
    dv = np.zeros((Tk, Hkv, d))
    allk = np.arange(Tk)
    for h in heads:
        g = _head_group(h, Hq, Hkv)
        mg = _mask_group(spec, h, Hq)
        for r0 in range(0, len(rows_all), ROW_BLOCK):
            rr = rows_all[r0:r0 + ROW_BLOCK]
            if o is None or lse is None:
                ob, lb = fwd_rows(q, k, v, spec, scale, h, rr)
            else:
                ob = to_f64(o)[rr, h, :]
                lb = to_f64(lse)[h, rr]
            M = _masks.allowed(spec, rr, allk, mg)
            cols = np.nonzero(M.any(axis=0))[0]
            if cols.size == 0:
                continue
            Mc = M[:, cols]
            S = scale * (q[rr, h, :] @ k[cols, g, :].T)
            fin = np.isfinite(lb)
            lsafe = np.where(fin, lb, 0.0)
            P = np.where(Mc & fin[:, None], np.exp(np.where(Mc, S, 0.0) - lsafe[:, None]), 0.0)
            dob = do[rr, h, :]
            D = (dob * ob).sum(axis=1)
            dP = dob @ v[cols, g, :].T
            dS = P * (dP - D[:, None])
            if "dq" in want:
                dq[r0:r0 + len(rr), h, :] = scale * (dS @ k[cols, g, :])
            if "dk" in want:
                dk[cols, g, :] += scale * (dS.T @ q[rr, h, :])
            if "dv" in want:
                dv[cols, g, :] += P.T @ dob
    return {"dq": dq, "dk": dk, "dv": dv}


def attn_bwd_keys(q, k, v, do, spec, scale, keys, kv_heads=None, rows=None):
    """dK, dV at chosen key columns only: ([len(keys), len(kv_heads), d] each).

    The same definition as attn_bwd restricted to the columns j in `keys`:
    dK_j = scale * sum_{h in group} sum_i dS^h_ij q^h_i and
    dV_j = sum_{h in group} sum_i P^h_ij dO^h_i.  Every query row of the
    group's heads that sees one of the keys contributes (only the rows in
    `rows`, if given: the sums split over disjoint row sets); each such row's
    O and LSE (hence P and D) come from the oracle's own forward over all of
    that row's keys.  Rows that see none of the chosen keys contribute
    nothing and are skipped.
    """
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    R = Hq // Hkv
    keys = np.asarray(keys, dtype=np.int64)
    kv_heads = list(range(Hkv)) if kv_heads is None else list(kv_heads)
    dk = np.zeros((len(keys), len(kv_heads), d))
    dv = np.zeros((len(keys), len(kv_heads), d))
    for gi, g in enumerate(kv_heads):
        for h in range(g * R, (g + 1) * R):
            mg = _mask_group(spec, h, Hq)
            rows_all = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
            for r0 in range(0, len(rows_all), ROW_BLOCK):
                rr = rows_all[r0:r0 + ROW_BLOCK]
                Mk = _masks.allowed(spec, rr, keys, mg)
                sel = Mk.any(axis=1)
                if not sel.any():
                    continue
                rs, Mk = rr[sel], Mk[sel]
                ob, lb = fwd_rows(q, k, v, spec, scale, h, rs)  # every row here has a key, so lb is finite
                S = scale * (q[rs, h, :] @ k[keys, g, :].T)
                P = np.where(Mk, np.exp(np.where(Mk, S, 0.0) - lb[:, None]), 0.0)
                dob = do[rs, h, :]
                D = (dob * ob).sum(axis=1)
                dS = P * (dob @ v[keys, g, :].T - D[:, None])
                dk[:, gi, :] += scale * (dS.T @ q[rs, h, :])
                dv[:, gi, :] += P.T @ dob
    return dk, dv
