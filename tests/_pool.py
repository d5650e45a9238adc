"""Run the oracle head by head in a process pool (test helper).

Full-size parity needs the fp64 oracle over whole heads; one head is
independent of another (a KV head's dK / dV is the sum of its query heads'
contributions), so each task gets one query head's slice of the inputs and
the caller sums or stacks the results.  Workers are started with "spawn" and
import only numpy and the oracle: they never touch the GPU.
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


def _f64(x):
    if hasattr(x, "detach"):
        return x.detach().float().numpy().astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def _head_task(args):
    """One query head: O [T, d], LSE [T], dQ [T, d] and this head's dK / dV contribution [Tk, d]."""
    q, k, v, do, spec, scale, want_bwd = args
    from oracle import attention as A
    O, L = A.attn_fwd(q[:, None], k[:, None], v[:, None], spec, scale)
    out = {"o": O[:, 0], "lse": L[0]}
    if want_bwd:
        g = A.attn_bwd(q[:, None], k[:, None], v[:, None], do[:, None], spec, scale)
        out.update(dq=g["dq"][:, 0], dk=g["dk"][:, 0], dv=g["dv"][:, 0])
    return out


def _keys_task(args):
    q, k, v, do, spec, scale, keys = args
    from oracle import attention as A
    dk, dv = A.attn_bwd_keys(q[:, None], k[:, None], v[:, None], do[:, None], spec, scale, keys)
    return dk[:, 0], dv[:, 0]


def _run(fn, tasks):
    if len(tasks) == 1:
        return [fn(tasks[0])]
    out = []
    with mp.get_context("spawn").Pool(n_workers(len(tasks))) as pool:
        for i, r in enumerate(pool.imap(fn, tasks, chunksize=1)):
            out.append(r)
            print(f"  oracle head task {i + 1}/{len(tasks)} done", flush=True)
    return out


def head_spec(spec, h, Hq):
    """The mask of query head h as a one-group spec (block-sparse keep sets are per mask group)."""
    if spec.keep is None or spec.keep.shape[0] == 1:
        return spec
    import dataclasses
    G = spec.keep.shape[0]
    mg = h // (Hq // G)
    return dataclasses.replace(spec, keep=spec.keep[mg:mg + 1])


def oracle_heads(q, k, v, do, spec, scale, heads, bwd=True):
    """Oracle results for the given query heads: o [T, len, d], lse [len, T], dq [T, len, d], and
    dk / dv [Tk, Hkv, d] holding the listed heads' contributions (complete for a KV head when
    every query head of its group is listed)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    Hq, Hkv = q.shape[1], k.shape[1]
    R = Hq // Hkv
    tasks = [(q[:, h], k[:, h // R], v[:, h // R], do[:, h], head_spec(spec, h, Hq), scale, bwd) for h in heads]
    res = _run(_head_task, tasks)
    out = {"o": np.stack([r["o"] for r in res], axis=1), "lse": np.stack([r["lse"] for r in res], axis=0)}
    if bwd:
        out["dq"] = np.stack([r["dq"] for r in res], axis=1)
        dk = np.zeros(k.shape)
        dv = np.zeros(v.shape)
        for h, r in zip(heads, res):
            dk[:, h // R] += r["dk"]
            dv[:, h // R] += r["dv"]
        out["dk"], out["dv"] = dk, dv
    return out


def oracle_keys(q, k, v, do, spec, scale, keys, kv_head):
    """dK, dV [len(keys), d] of KV head kv_head at the given key columns (all its query heads)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    Hq, Hkv = q.shape[1], k.shape[1]
    R = Hq // Hkv
    heads = range(kv_head * R, (kv_head + 1) * R)
    tasks = [(q[:, h], k[:, kv_head], v[:, kv_head], do[:, h], head_spec(spec, h, Hq), scale, np.asarray(keys))
             for h in heads]
    res = _run(_keys_task, tasks)
    return sum(r[0] for r in res), sum(r[1] for r in res)
