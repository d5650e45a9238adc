"""Run the oracle over (query head, row range) tasks in a process pool (test helper).

Full-size parity needs the fp64 oracle over whole heads.  One head is
independent of another, and within a head the query rows are independent
(each row's O, LSE and dQ, and its share of dK / dV, which add up over
disjoint row sets), so each task gets one query head's slice of the inputs
and a range of rows, and the caller stacks or sums the results.  Workers are
started with "spawn", use one BLAS thread each (the pool spreads the tasks
over the cores), import only numpy and the oracle, and never touch the GPU.
"""
import multiprocessing as mp
import os

import numpy as np


def n_workers(n_tasks):
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return max(1, min(n_tasks, cores, 16))


def _init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def _f64(x):
    if hasattr(x, "detach"):
        return x.detach().float().numpy().astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def _head_task(args):
    """Rows `rows` of one query head: O, LSE, dQ of those rows and their dK / dV contribution [Tk, d]."""
    q, k, v, do, spec, scale, rows, want_bwd = args
    from oracle import attention as A
    O, L = A.attn_fwd(q[:, None], k[:, None], v[:, None], spec, scale, rows=rows)
    out = {"o": O[:, 0], "lse": L[0]}
    if want_bwd:
        g = A.attn_bwd(q[:, None], k[:, None], v[:, None], do[:, None], spec, scale, rows=rows)
        out.update(dq=g["dq"][:, 0], dk=g["dk"][:, 0], dv=g["dv"][:, 0])
    return out


def _keys_task(args):
    q, k, v, do, spec, scale, keys, rows = args
    from oracle import attention as A
    dk, dv = A.attn_bwd_keys(q[:, None], k[:, None], v[:, None], do[:, None], spec, scale, keys, rows=rows)
    return dk[:, 0], dv[:, 0]


def _run(fn, tasks):
    if len(tasks) == 1:
        return [fn(tasks[0])]
    out = []
    with mp.get_context("spawn").Pool(n_workers(len(tasks)), initializer=_init) as pool:
        for i, r in enumerate(pool.imap(fn, tasks, chunksize=1)):
            out.append(r)
            if (i + 1) % 8 == 0 or i + 1 == len(tasks):
                print(f"  oracle tasks {i + 1}/{len(tasks)} done", flush=True)
    return out


def head_spec(spec, h, Hq):
    """The mask of query head h as a one-group spec (block-sparse keep sets are per mask group)."""
    if spec.keep is None or spec.keep.shape[0] == 1:
        return spec
    import dataclasses
    G = spec.keep.shape[0]
    mg = h // (Hq // G)
    return dataclasses.replace(spec, keep=spec.keep[mg:mg + 1])


def _row_chunks(T, n):
    edges = np.linspace(0, T, n + 1).astype(np.int64)
    return [np.arange(edges[i], edges[i + 1]) for i in range(n) if edges[i + 1] > edges[i]]


def _chunks_per_head(n_heads, T):
    """Row ranges per head so that the tasks fill the pool (at most 16 workers)."""
    return max(1, min(T // 256, -(-16 // max(1, n_heads))))


def oracle_heads(q, k, v, do, spec, scale, heads, bwd=True):
    """Oracle results for the given query heads: o [T, len, d], lse [len, T], dq [T, len, d], and
    dk / dv [Tk, Hkv, d] holding the listed heads' contributions (complete for a KV head when
    every query head of its group is listed)."""
    heads = list(heads)
    Hq, Hkv = q.shape[1], k.shape[1]
    R = Hq // Hkv
    T = q.shape[0]
    chunks = _row_chunks(T, _chunks_per_head(len(heads), T))
    kf = {g: (_f64(k[:, g]), _f64(v[:, g])) for g in sorted({h // R for h in heads})}
    tasks, index = [], []
    for hi, h in enumerate(heads):
        qh, dh = _f64(q[:, h]), _f64(do[:, h])
        for rows in chunks:
            tasks.append((qh, *kf[h // R], dh, head_spec(spec, h, Hq), scale, rows, bwd))
            index.append((hi, h, rows))
    res = _run(_head_task, tasks)
    d = q.shape[2]
    out = {"o": np.zeros((T, len(heads), d)), "lse": np.full((len(heads), T), -np.inf)}
    if bwd:
        out.update(dq=np.zeros((T, len(heads), d)), dk=np.zeros(k.shape), dv=np.zeros(v.shape))
    for (hi, h, rows), r in zip(index, res):
        out["o"][rows, hi] = r["o"]
        out["lse"][hi, rows] = r["lse"]
        if bwd:
            out["dq"][rows, hi] = r["dq"]
            out["dk"][:, h // R] += r["dk"]
            out["dv"][:, h // R] += r["dv"]
    return out


def oracle_keys(q, k, v, do, spec, scale, keys, kv_head):
    """dK, dV [len(keys), d] of KV head kv_head at the given key columns (all its query heads)."""
    Hq, Hkv = q.shape[1], k.shape[1]
    R = Hq // Hkv
    T = q.shape[0]
    kg, vg = _f64(k[:, kv_head]), _f64(v[:, kv_head])
    chunks = _row_chunks(T, _chunks_per_head(R, T))
    tasks = []
    for h in range(kv_head * R, (kv_head + 1) * R):
        qh, dh = _f64(q[:, h]), _f64(do[:, h])
        for rows in chunks:
            tasks.append((qh, kg, vg, dh, head_spec(spec, h, Hq), scale, np.asarray(keys), rows))
    res = _run(_keys_task, tasks)
    return sum(r[0] for r in res), sum(r[1] for r in res)
