#!/usr/bin/env python3
"""Benchmark of the masked-attention hot path on one MI355X.

Metric: effective attention TFLOP/s, counting only unmasked FLOPs, for the
forward and for forward + backward, against the bf16 MFMA peak.  One step is
one pass of the whole path over the workload: forward (O, LSE), then the
backward's delta pre-pass, dK/dV kernel and dQ kernel.  Inputs are seeded
synthetic bf16 N(0,1) tensors already resident in HBM; the mask plan is
compiled and uploaded before timing (static masks are fixed before training,
LongCA-bench section 2.1.1).  Timing follows the pages' protocol of warm-up
steps before timed steps (appendix A.4: 5 warm-ups, 20 steps).

Default workload: CAUSAL, one packed sequence of 32768 tokens, GQA 64 query
heads : 8 KV heads, head dim 128.  Prints one JSON line.

`--suite` instead runs every workload family of the path -- the twelve static
masks at 32K, uniform and variable block-sparse masks at 32K and 128K, and
ring-step shares at their 8K x 8K shape -- and prints one JSON line per
workload.

`--gpus N` with N > 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective attention TFLOP/s fwd and fwd+bwd (unmasked FLOPs) vs bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNEL_SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "attn_dkdv.hip", "attn_dkdv.hpp", "attn_dkdv256.hip", "ring.hip",
                  "blockmask.hip", "kernel_common.hpp", "plan.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
NAMES = ["fwd", "delta", "dkdv", "dq"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seq", type=int, default=32768)
    ap.add_argument("--hq", type=int, default=64)
    ap.add_argument("--hkv", type=int, default=8)
    ap.add_argument("--d", type=int, default=128)
    ap.add_argument("--mask", default="CAUSAL")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-rows", type=int, default=1024, help="query rows in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fwd-only", action="store_true", help="time only the forward (profiling aid)")
    ap.add_argument("--suite", action="store_true", help="run every workload family, one JSON line each")
    ap.add_argument("--only", default="", help="with --suite: comma-separated substrings of workload names")
    ap.add_argument("--runs", type=int, default=2,
                    help="timed runs (warm-up + steps each) of a single-sequence workload; the line reports the "
                         "median (the pages' protocol: two runs)")
    ap.add_argument("--doc-seeds", type=int, default=1,
                    help="with --suite: document-length samples per multi-sequence mask (median reported)")
    ap.add_argument("--memory", action="store_true",
                    help="peak device memory of fwd and fwd+bwd over sequence lengths 1K..48K (one JSON line each)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (HBM byte-counter calibration) and exit")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of the kernel sources and the device build flags they are compiled with."""
    from mask_aware_dense_amd import build as mad_build
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mask_aware_dense_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    dev_flags = [f.replace(mad_build.ROOT, "") for f in mad_build.flags()]  # no absolute paths
    h.update(repr((dev_flags, sorted(mad_build.SOURCE_FLAGS.items()))).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources and this workload; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else float(k["hbm_bytes_per_launch"])


_WORKER = {}


def _pool_init(seed, T, Hq, Hkv, d, barrier):
    """Pool worker start-up (untimed): one BLAS thread (the pool spreads the heads over the cores) and
    the workload's inputs regenerated from the seed, so tasks carry only a head index.  It never
    raises (a failing initializer would make the pool start replacement workers without end): a
    failure is kept and reported by the worker's first task."""
    try:
        try:
            from threadpoolctl import threadpool_limits
            threadpool_limits(1)
        except ImportError:
            pass
        import torch
        torch.set_num_threads(1)
        from mad_inputs import grad_out, qkv
        _WORKER["qkv"] = qkv(seed, T, T, Hq, Hkv, d)
        _WORKER["do"] = grad_out(seed, T, Hq, d)
    except Exception as e:  # noqa: BLE001
        _WORKER["error"] = repr(e)
    try:
        barrier.wait(timeout=600)
    except Exception:  # noqa: BLE001
        pass


def _cpu_head_task(a):
    """The oracle, as it stands, on one query head: forward of the sampled rows and their share of the
    backward."""
    h, spec, scale, rows = a
    if "error" in _WORKER:
        raise RuntimeError(f"oracle worker start-up failed: {_WORKER['error']}")
    from oracle import attention as A
    q, k, v = _WORKER["qkv"]
    R = q.shape[1] // k.shape[1]
    qh, kh, vh, doh = (A.to_f64(x) for x in (q[:, h:h + 1], k[:, h // R:h // R + 1], v[:, h // R:h // R + 1],
                                             _WORKER["do"][:, h:h + 1]))
    t0 = time.perf_counter()
    A.attn_fwd(qh, kh, vh, spec, scale, rows=rows)
    A.attn_bwd(qh, kh, vh, doh, spec, scale, rows=rows)
    return time.perf_counter() - t0


def _timed_pool(args, spec, scale, rows, cores):
    """Wall time of the oracle over every head on `cores` worker processes (start-up excluded)."""
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(cores)
    with ctx.Pool(cores, initializer=_pool_init,
                  initargs=(args.seed, args.seq, args.hq, args.hkv, args.d, barrier)) as pool:
        pool.map(time.sleep, [0.05] * cores, chunksize=1)  # returns once the workers have started up
        t0 = time.perf_counter()
        pool.map(_cpu_head_task, [(h, spec, scale, rows) for h in range(args.hq)], chunksize=1)
        return time.perf_counter() - t0


def cpu_baseline(args, q, k, v, do, spec, scale):
    """Oracle (fp64 numpy, as it stands) on a bounded sample of the same workload, heads spread over a
    process pool on every host core this process may use; plus the tiny reference configuration
    (T=1024, MHA 4:4, d=64, FULL and CAUSAL) in full."""
    from oracle import attention as A
    from oracle import masks as M
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng([args.seed, 9])
    rows = np.sort(rng.choice(args.seq, size=min(args.cpu_rows, args.seq), replace=False))
    workers = min(cores, args.hq)
    dt = _timed_pool(args, spec, scale, rows, workers)
    pairs = int(M.allowed(spec, rows, np.arange(args.seq)).sum()) * args.hq
    flop = 14.0 * args.d * pairs
    # the tiny reference configuration in full (forward, then forward + backward)
    from mad_inputs import grad_out, qkv
    tiny = {}
    for mask in ("FULL", "CAUSAL"):
        tq, tk, tv = (A.to_f64(x) for x in qkv(0, 1024, 1024, 4, 4, 64))
        tdo = A.to_f64(grad_out(0, 1024, 4, 64))
        tspec = M.MaskSpec(mask, 1024, 1024)
        t0 = time.perf_counter()
        A.attn_fwd(tq, tk, tv, tspec, 0.125)
        t_f = time.perf_counter() - t0
        A.attn_bwd(tq, tk, tv, tdo, tspec, 0.125)
        t_fb = time.perf_counter() - t0
        tp = M.pair_count(tspec) * 4
        tiny[mask] = {"fwd_s": t_f, "fwdbwd_s": t_fb, "fwd_gflops": 4.0 * 64 * tp / t_f / 1e9,
                      "fwdbwd_gflops": 14.0 * 64 * tp / t_fb / 1e9}
    return {
        "value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(workers), "kind": "oracle",
        "seconds": dt,
        "sample": f"{len(rows)} seeded query rows x {args.hq} heads of the same workload, fp64 forward + "
                  f"backward (those rows' share of dQ, dK, dV), one head per task on a pool of {workers} "
                  f"processes (one per core this process may use) with one BLAS thread each; effective "
                  f"FLOPs 14*d*pairs",
        "tiny_reference_full": {"config": "T=1024, MHA 4:4, d=64, scale 1/8, seed 0; whole forward and "
                                          "forward + backward in this process (BLAS at its default threads)",
                                **tiny},
    }


class Runner:
    """Times the path on one plan and one set of device tensors."""

    def __init__(self, torch, mad, plan, Tq, Tk, Hq, Hkv, d, seed):
        from mad_inputs import grad_out, qkv
        self.torch, self.mad, self.plan = torch, mad, plan
        dev = torch.device("cuda", 0)
        q, k, v = qkv(seed, Tq, Tk, Hq, Hkv, d)
        do = grad_out(seed, Tq, Hq, d)
        self.host = (q, k, v, do)
        self.q, self.k, self.v, self.do = (x.to(dev) for x in (q, k, v, do))
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((Hq, Tq), dtype=torch.float32, device=dev)
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        self.ws = torch.empty(mad.bwd_workspace_bytes(plan, Tq, Tk, Hq, Hkv, d), dtype=torch.uint8, device=dev)
        self.fws = torch.empty(mad.FWD_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
        self.scale = 1.0 / np.sqrt(d)
        self.stream = torch.cuda.current_stream()

    def use_plan(self, plan, Tq, Tk, Hq, Hkv, d):
        """Another plan over the same shapes (the inputs stay); the workspace grows if needed."""
        self.plan = plan
        need = self.mad.bwd_workspace_bytes(plan, Tq, Tk, Hq, Hkv, d)
        if need > self.ws.numel():
            self.ws = self.torch.empty(need, dtype=self.torch.uint8, device=self.ws.device)

    def step(self, fwd_only=False, evs=None):
        mad, s = self.mad, self.stream
        if evs is not None:
            evs[0].record(s)
        mad.attn_fwd(self.plan, self.q, self.k, self.v, self.o, self.lse, self.scale, s, workspace=self.fws)
        if evs is not None:
            evs[1].record(s)
        if fwd_only:
            return
        for i, ph in enumerate((mad.BWD_DELTA, mad.BWD_DKDV, mad.BWD_DQ)):
            mad.attn_bwd_phases(self.plan, self.q, self.k, self.v, self.o, self.do, self.lse, self.dq, self.dk,
                                self.dv, self.ws, self.scale, ph, s)
            if evs is not None:
                evs[2 + i].record(s)

    def time(self, steps, warmup, fwd_only=False):
        """Returns (wall seconds for `steps` steps, per-kernel mean ms, per-kernel median ms)."""
        torch = self.torch
        for _ in range(warmup):
            self.step(fwd_only)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            self.step(fwd_only, evs[s])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        nk = 1 if fwd_only else 4
        per = np.array([[evs[s][i].elapsed_time(evs[s][i + 1]) for i in range(nk)] for s in range(steps)])
        mean = {NAMES[i]: float(np.mean(per[:, i])) for i in range(nk)}
        med = {NAMES[i]: float(np.median(per[:, i])) for i in range(nk)}
        return wall, mean, med


def roofline(kern_ms, pairs, d, T, Hq, workload):
    """Roofline entry of the dominant kernel (largest mean time).

    Algorithmic work per launch: forward 4d FLOP per unmasked (query, key,
    head) pair; dK/dV kernel 8d (its S, dP, dV, dK products); dQ kernel 2d
    (its dQ product -- its S and dP are recomputed, not algorithmic); the
    delta pre-pass is HBM-bound (reads O and dO, writes two fp32 rows).
    """
    alg = {"fwd": 4.0 * d * pairs, "dkdv": 8.0 * d * pairs, "dq": 2.0 * d * pairs}
    dom = max(kern_ms, key=kern_ms.get)
    traffic = measured_traffic(dom, workload)
    if dom == "delta":
        bytes_ = 2.0 * 2 * T * Hq * d + 8.0 * T * Hq
        ach = bytes_ / (kern_ms[dom] * 1e-3) / 1e9
        return {"kernel": "delta", "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS, "traffic": traffic}
    ach = alg[dom] / (kern_ms[dom] * 1e-3) / 1e12
    return {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS, "traffic": traffic}


# ---------------------------------------------------------------------------
# Workload suite
# ---------------------------------------------------------------------------
def suite_workloads(seed):
    """(name, builder) pairs; a builder returns (plan, Tq, Tk, Hq, Hkv, d, config dict)."""
    from mad_inputs import answer_lengths, block_scores, doc_lengths, variable_block_sizes
    T = 32768
    out = []

    def static(pattern, **kw):
        def build(mad):
            sl = mad.mask_slices(pattern, T, **kw)
            return mad.mask_compile(sl, T, T), T, T, 64, 8, 128, {"mask": pattern, "seq_len": T, **{
                k: (v if not isinstance(v, (list, np.ndarray)) else
                    (f"{len(v)} documents" if k == "doc_lens" else f"sampled {list(v)}")) for k, v in kw.items()}}
        return build

    docs = [int(x) for x in doc_lengths(seed, T)]
    for pattern, kw in [
        ("FULL", {}), ("CAUSAL", {}), ("SLIDING_WINDOW", {"window": 4096}),
        ("FULL_DOCUMENT", {"doc_lens": docs}), ("CAUSAL_DOCUMENT", {"doc_lens": docs}),
        ("SLIDING_WINDOW_CAUSAL_DOCUMENT", {"window": 4096, "doc_lens": docs}),
        ("PREFIX_LM", {}),
        ("SHARED_QUESTION", {"question": 2048, "answer_lens": [int(x) for x in answer_lengths(seed, T - 2048, 4)]}),
        ("GLOBAL_SLIDING", {"global_len": 256, "window": 2048}), ("CAUSAL_BLOCKWISE", {"block": 2048}),
        ("BLOCK_CAUSAL_DOCUMENT", {"block": 1024, "doc_lens": docs}), ("PREFIX_LM_DOCUMENT", {"doc_lens": docs}),
        ("CAUSAL_BLOCKWISE_LAST", {"block": 2048}),
        ("BLOCK_CAUSAL_DOCUMENT_GLOBAL", {"block": 1024, "doc_lens": docs}),
    ]:
        out.append((f"{pattern} 32K GQA 64:8", static(pattern, **kw)))

    def head_dim(pattern, d):
        def build(mad):
            return mad.mask_compile(mad.mask_slices(pattern, T), T, T), T, T, 64, 8, d, {
                "mask": pattern, "seq_len": T}
        return build

    for d in (64, 256):
        out.append((f"CAUSAL 32K GQA 64:8 d={d}", head_dim("CAUSAL", d)))

    # the regular masks at the other totals and head layouts the workloads name
    def sized(pattern, T_, Hq, Hkv, **kw):
        def build(mad):
            kw2 = dict(kw)
            if "doc_lens" in kw2:
                kw2["doc_lens"] = [int(x) for x in doc_lengths(seed, T_)]
            sl = mad.mask_slices(pattern, T_, **kw2)
            return mad.mask_compile(sl, T_, T_), T_, T_, Hq, Hkv, 128, {
                "mask": pattern, "seq_len": T_, **({"window": kw["window"]} if "window" in kw else {}),
                **({"doc_lens": f"{len(kw2['doc_lens'])} documents"} if "doc_lens" in kw2 else {})}
        return build

    for pattern, T_, Hq, Hkv, kw in [
        ("CAUSAL", 8192, 64, 8, {}), ("CAUSAL", 49152, 64, 8, {}), ("CAUSAL", 32768, 64, 64, {}),
        ("FULL", 16384, 64, 64, {}), ("SLIDING_WINDOW", 49152, 64, 64, {"window": 4096}),
        ("CAUSAL_DOCUMENT", 49152, 64, 8, {"doc_lens": True}), ("FULL_DOCUMENT", 16384, 64, 64, {"doc_lens": True}),
    ]:
        heads = "MHA 64:64" if Hq == Hkv else f"GQA {Hq}:{Hkv}"
        out.append((f"{pattern} {T_ // 1024}K {heads}", sized(pattern, T_, Hq, Hkv, **kw)))

    def varlen_continuation():
        # a batch of the same 32K of documents as keys; each sequence's queries are the
        # last half of its tokens (a chunk that continues a cached prefix), causal,
        # bottom-right aligned
        def build(mad):
            lk = np.asarray(docs, dtype=np.int64)
            lq = lk - lk // 2
            cq = np.concatenate([[0], np.cumsum(lq)])
            ck = np.concatenate([[0], np.cumsum(lk)])
            sl = mad.varlen_slices(cq, ck, causal=True, bottom_right=True)
            Tq, Tk = int(cq[-1]), int(ck[-1])
            return mad.mask_compile(sl, Tq, Tk), Tq, Tk, 64, 8, 128, {
                "mask": "VARLEN causal bottom-right", "seq_len_q": Tq, "seq_len_k": Tk,
                "batch": len(docs), "queries": "last half of each sequence"}
        return build

    out.append(("VARLEN continuation 32K keys GQA 64:8", varlen_continuation()))

    def sparse(S, Hq, Hkv, b, pct, variable):
        def build(mad):
            G = Hkv  # one keep set per KV-head group (per head for MHA)
            if variable:
                sizes = variable_block_sizes(seed, S, 32, 256)
                edges = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
            else:
                edges = np.arange(0, S + 1, b, dtype=np.int32)
            n = len(edges) - 1
            keep = mad.block_topk(block_scores(seed, G, n, n), pct)
            plan = mad.sparse_plan(G, edges, edges, keep)
            return plan, S, S, Hq, Hkv, 128, {
                "mask": "VARIABLE_BLOCK_SPARSE" if variable else "BLOCK_SPARSE", "seq_len": S,
                "block": "U{32..256}" if variable else b, "sparsity": pct / 100.0, "keep_groups": G}
        return build

    for S, Hq, Hkv, b, pct, var in [
        (32768, 64, 8, 128, 20, False), (32768, 64, 8, 128, 50, False), (32768, 64, 8, 128, 80, False),
        (32768, 64, 8, 64, 50, False), (32768, 64, 64, 64, 80, False), (32768, 64, 8, 0, 50, True),
        (131072, 64, 8, 128, 20, False), (131072, 64, 64, 64, 20, False),
    ]:
        tag = "variable" if var else f"b{b}"
        heads = "MHA 64:64" if Hq == Hkv else f"GQA {Hq}:{Hkv}"
        out.append((f"BLOCK_SPARSE {S // 1024}K {heads} {tag} s{pct / 100:.1f}", sparse(S, Hq, Hkv, b, pct, var)))

    def ring(layout, rank, source):
        def build(mad):
            C = 8192
            sl = mad.ring_step_slices(layout, 12, C, rank, source)
            return mad.mask_compile(sl, C, C), C, C, 64, 8, 128, {
                "mask": "RING_STEP", "layout": layout, "n_ranks": 12, "rank": rank, "source": source,
                "chunk": C}
        return build

    for layout, rank, source in [("contiguous", 11, 0), ("contiguous", 11, 11), ("headtail", 0, 0),
                                 ("headtail", 0, 5)]:
        out.append((f"RING_STEP {layout} r{rank} s{source} 8K", ring(layout, rank, source)))
    return out


def multi_sequence(name):
    """Workloads whose structure depends on sampled lengths (documents, varlen sequences, the answers
    of a Shared Question mask): the pages time them over 30 independently sampled runs."""
    return "DOCUMENT" in name or "VARLEN" in name or "SHARED_QUESTION" in name


def run_suite(args, torch, mad):
    only = [s.strip() for s in args.only.split(",") if s.strip()]
    n_seeds = max(1, args.doc_seeds)
    other_seeds = [dict(suite_workloads(args.seed + i)) for i in range(1, n_seeds)]
    for name, build in suite_workloads(args.seed):
        if only and not any(o in name for o in only):
            continue
        print(f"workload: {name}", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        plan, Tq, Tk, Hq, Hkv, d, cfg = build(mad)
        plan_s = time.perf_counter() - t0
        plan.upload()
        st = plan.stats(0)
        G = len(st["pairs"])
        pairs = int(sum(int(x) for x in st["pairs"]) * (Hq // G))
        r = Runner(torch, mad, plan, Tq, Tk, Hq, Hkv, d, args.seed)
        wall, mean, med = r.time(args.steps, args.warmup)
        t_fwd = mean["fwd"] * 1e-3
        fwdbwd = 14.0 * d * pairs * args.steps / wall / 1e12
        seeds = None
        if n_seeds > 1 and multi_sequence(name):
            # the same mask family over further document-length samples, each with its own plan
            # and the same warm-up and step counts; the line reports the median
            vals = [fwdbwd]
            n2 = args.steps
            for extra in other_seeds:
                p2, Tq2, Tk2, Hq2, Hkv2, d2, _ = extra[name](mad)
                p2.upload()
                st2 = p2.stats(0)
                pr2 = int(sum(int(x) for x in st2["pairs"]) * (Hq2 // len(st2["pairs"])))
                if (Tq2, Tk2) == (Tq, Tk):
                    r2 = r
                    r2.use_plan(p2, Tq2, Tk2, Hq2, Hkv2, d2)
                else:  # a varlen sample of another total length
                    r2 = Runner(torch, mad, p2, Tq2, Tk2, Hq2, Hkv2, d2, args.seed)
                w2, _, _ = r2.time(n2, args.warmup)
                vals.append(14.0 * d2 * pr2 * n2 / w2 / 1e12)
                del r2, p2
            seeds = {"n": len(vals), "median": float(np.median(vals)), "min": float(min(vals)),
                     "max": float(max(vals)), "first_sample": fwdbwd}
            fwdbwd = seeds["median"]
        runs = None
        if args.runs > 1 and not multi_sequence(name):
            # a single-sequence mask: the same timed steps repeated, the line reports the median
            vals = [fwdbwd]
            for _ in range(args.runs - 1):
                w2, _, _ = r.time(args.steps, args.warmup)
                vals.append(14.0 * d * pairs * args.steps / w2 / 1e12)
            runs = {"n": len(vals), "median": float(np.median(vals)), "min": float(min(vals)),
                    "max": float(max(vals))}
            fwdbwd = runs["median"]
        rec = {
            "workload": name, "metric": METRIC, "unit": "TFLOP/s", "value": fwdbwd,
            "fwd_tflops": 4.0 * d * pairs / t_fwd / 1e12, "fwdbwd_frac_peak": fwdbwd / PEAK_BF16_TFLOPS,
            "ms_per_step": wall * 1e3 / args.steps, "kernel_ms_mean": mean, "kernel_ms_median": med,
            "unmasked_pairs": pairs, "density": pairs / (float(Tq) * Tk * Hq), "plan_compile_s": plan_s,
            "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": name, **cfg, "heads_q": Hq, "heads_kv": Hkv, "head_dim": d},
            "roofline": roofline(mean, pairs, d, Tq, Hq, name),
            "delta_hbm_gbs": (2.0 * 2 * Tq * Hq * d + 8.0 * Tq * Hq) / (mean["delta"] * 1e-3) / 1e9,
            "kernel_source_hash": kernel_source_hash(),
        }
        if seeds:
            rec["doc_seeds"] = seeds
        if runs:
            rec["runs"] = runs
        print(json.dumps(rec), flush=True)
        del r, plan
        torch.cuda.empty_cache()
    for S, Hq, Hkv, G, b, pct in [(32768, 64, 8, 8, 128, 50), (131072, 64, 8, 8, 128, 80), (32768, 64, 64, 64, 64, 80)]:
        heads = "MHA 64:64" if Hq == Hkv else f"GQA {Hq}:{Hkv}"
        name = f"DYNAMIC BLOCK_SPARSE {S // 1024}K {heads} b{b} s{pct / 100:.1f}: GPU scores + top-k, plan, attention"
        if only and not any(o in name for o in only):
            continue
        print(f"workload: {name}", file=sys.stderr, flush=True)
        print(json.dumps(dynamic_sparse(args, torch, mad, S, Hq, Hkv, G, b, pct, name)), flush=True)
        torch.cuda.empty_cache()
    for layout, rank in [("headtail", 0), ("contiguous", 11)]:
        name = f"RING 12x8K {layout} rank {rank}: all steps + merge, backward"
        if only and not any(o in name for o in only):
            continue
        print(f"workload: {name}", file=sys.stderr, flush=True)
        print(json.dumps(ring_share(args, torch, mad, layout, 12, 8192, rank, name)), flush=True)
        torch.cuda.empty_cache()


def dynamic_sparse(args, torch, mad, S, Hq, Hkv, G, b, pct, name, d=128):
    """A dynamic block-sparse mask made from Q and K on the GPU (pooled block scores, top-k), the
    plan compiled on the GPU from its keep bitmap, then attention under it.  The host compile of
    the same bitmap (copied back) is timed beside it."""
    dev = torch.device("cuda", 0)
    edges = np.arange(0, S + 1, b, dtype=np.int32)
    n = len(edges) - 1
    r = None
    ws = torch.empty(mad.block_mask_workspace_bytes(G, Hkv, n, n, d), dtype=torch.uint8, device=dev)
    keep = torch.empty((G, n, (n + 63) // 64), dtype=torch.int64, device=dev)
    e_d = torch.from_numpy(edges).to(dev)
    from mad_inputs import qkv
    q, k, _ = qkv(args.seed, S, S, Hq, Hkv, d)
    qd, kd = q.to(dev), k.to(dev)
    scale = 1.0 / np.sqrt(d)
    for _ in range(2):
        mad.block_mask(qd, kd, G, e_d, e_d, pct, scale, keep, ws)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(5):
        mad.block_mask(qd, kd, G, e_d, e_d, pct, scale, keep, ws)
    ev[1].record()
    torch.cuda.synchronize()
    gen_ms = ev[0].elapsed_time(ev[1]) / 5
    t0 = time.perf_counter()
    kw = keep.cpu().numpy().view(np.uint64)
    hplan = mad.sparse_plan(G, edges, edges, kw)
    hplan.upload()
    plan_s = time.perf_counter() - t0
    del hplan
    plan = mad.sparse_plan_device(G, edges, edges, keep)  # warm-up
    torch.cuda.synchronize()
    del plan
    t0 = time.perf_counter()
    for _ in range(5):
        plan = mad.sparse_plan_device(G, edges, edges, keep)
        torch.cuda.synchronize()
        if _ < 4:
            del plan
    plan_gpu_ms = (time.perf_counter() - t0) / 5 * 1e3
    del qd, kd
    st = plan.stats(0)
    pairs = int(sum(int(x) for x in st["pairs"]) * (Hq // G))
    r = Runner(torch, mad, plan, S, S, Hq, Hkv, d, args.seed)
    wall, mean, med = r.time(args.steps, args.warmup)
    value = 14.0 * d * pairs * args.steps / wall / 1e12
    del r
    return {
        "workload": name, "metric": METRIC, "unit": "TFLOP/s", "value": value,
        "fwd_tflops": 4.0 * d * pairs / (mean["fwd"] * 1e-3) / 1e12, "fwdbwd_frac_peak": value / PEAK_BF16_TFLOPS,
        "ms_per_step": wall * 1e3 / args.steps, "kernel_ms_mean": mean, "kernel_ms_median": med,
        "mask_gen_gpu_ms": gen_ms, "plan_gpu_ms": plan_gpu_ms, "plan_host_s": plan_s, "unmasked_pairs": pairs,
        "density": pairs / (float(S) * S * Hq), "steps": args.steps, "warmup": args.warmup, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "mask": "BLOCK_SPARSE from pooled block scores", "seq_len": S, "block": b,
                   "sparsity": pct / 100.0, "keep_groups": G, "heads_q": Hq, "heads_kv": Hkv, "head_dim": d},
        "kernel_source_hash": kernel_source_hash(),
    }


def ring_share(args, torch, mad, layout, N, C, rank, name, Hq=64, Hkv=8, d=128):
    """One rank's whole ring share (every step's kernels, the K/V staging copies and the LSE merge
    in the forward; delta, every step's dK/dV and dQ kernels and the dQ rounding in the backward)."""
    from mad_inputs import grad_out, qkv
    dev = torch.device("cuda", 0)
    q, _, _ = qkv(args.seed, C, 1, Hq, Hkv, d)
    _, k, v = qkv(args.seed + 1, 1, N * C, Hq, Hkv, d)
    do = grad_out(args.seed, C, Hq, d)
    q, k, v, do = (x.to(dev) for x in (q, k, v, do))
    ring = mad.Ring(layout, N, C, rank, Hq, Hkv, d)
    info = ring.info()
    o = torch.empty_like(q)
    lse = torch.empty((Hq, C), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    scale = 1.0 / np.sqrt(d)
    s = torch.cuda.current_stream()

    def step(evs=None):
        if evs:
            evs[0].record(s)
        ring.fwd(q, k, v, o, lse, scale, s)
        if evs:
            evs[1].record(s)
        ring.bwd(q, k, v, o, do, lse, dq, dk, dv, scale, s)
        if evs:
            evs[2].record(s)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for x in range(args.steps):
        step(evs[x])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    pairs = info["pairs_per_head"] * Hq
    value = 14.0 * d * pairs * args.steps / wall / 1e12
    del ring
    return {
        "workload": name, "metric": METRIC, "unit": "TFLOP/s", "value": value,
        "fwd_tflops": 4.0 * d * pairs / (fwd * 1e-3) / 1e12, "fwdbwd_frac_peak": value / PEAK_BF16_TFLOPS,
        "ms_per_step": wall * 1e3 / args.steps, "kernel_ms_mean": {"fwd": fwd, "bwd": bwd},
        "unmasked_pairs": pairs, "density": pairs / (float(C) * N * C * Hq), "n_steps": info["n_steps"],
        "device_bytes": info["device_bytes"], "steps": args.steps, "warmup": args.warmup, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "mask": "CAUSAL over the ring", "layout": layout, "n_ranks": N, "chunk": C,
                   "rank": rank, "heads_q": Hq, "heads_kv": Hkv, "head_dim": d},
        "kernel_source_hash": kernel_source_hash(),
    }


def activation_model_bytes(b: int, s: int, h: int, d: int) -> int:
    """The pages' activation-memory model of a standard attention module (LongCA-bench appendix
    A.4.2): 11bshd + 5bhs^2 + 2bshd, read as bytes for batch b, sequence s, h heads of dim d."""
    return 11 * b * s * h * d + 5 * b * h * s * s + 2 * b * s * h * d


def _alloc_bytes(t) -> int:
    """Bytes torch's caching allocator counts for a tensor (sizes round up to 512 bytes)."""
    n = t.numel() * t.element_size()
    return (n + 511) // 512 * 512


def peak_memory_case(torch, mad, mask, T, Hq, Hkv, d, seed, kw=None):
    """Peak device memory of one forward and one forward+backward (appendix A.4.2): torch's allocator
    peak over the call's live tensors plus the plan's device block; beside it the allocator's count of
    the live tensors just before each call (equal to the peak if the call allocates nothing through
    torch), the tensors' own sizes (the allocator rounds each block up, by at most a segment
    remainder), and the free device memory before and after each call (unchanged if the library
    allocates nothing)."""
    from mad_inputs import grad_out, qkv
    dev = torch.device("cuda", 0)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    plan = mad.mask_compile(mad.mask_slices(mask, T, **(kw or {})), T, T)
    plan.upload()
    pb = plan.device_bytes()
    q, k, v = (x.to(dev) for x in qkv(seed, T, T, Hq, Hkv, d))
    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    fws = torch.empty(mad.FWD_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    scale = 1.0 / np.sqrt(d)
    torch.cuda.synchronize()
    live_f = torch.cuda.memory_allocated() - base  # the forward's tensors as the allocator counts them
    free0 = torch.cuda.mem_get_info()[0]
    mad.attn_fwd(plan, q, k, v, o, lse, scale, workspace=fws)
    torch.cuda.synchronize()
    free_f = torch.cuda.mem_get_info()[0]
    fwd_peak = torch.cuda.max_memory_allocated() - base + pb
    fwd_sum = sum(_alloc_bytes(t) for t in (q, k, v, o, lse, fws)) + pb
    do = grad_out(seed, T, Hq, d).to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(mad.bwd_workspace_bytes(plan, T, T, Hq, Hkv, d), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    live_b = torch.cuda.memory_allocated() - base
    free1 = torch.cuda.mem_get_info()[0]
    mad.attn_bwd(plan, q, k, v, o, do, lse, dq, dk, dv, ws, scale)
    torch.cuda.synchronize()
    bwd_peak = torch.cuda.max_memory_allocated() - base + pb
    bwd_sum = fwd_sum + sum(_alloc_bytes(t) for t in (do, dq, dk, dv, ws))
    free2 = torch.cuda.mem_get_info()[0]
    rec = {"fwd_peak_bytes": int(fwd_peak), "fwdbwd_peak_bytes": int(bwd_peak), "plan_device_bytes": int(pb),
           "fwd_live_plus_plan_bytes": int(live_f + pb), "fwdbwd_live_plus_plan_bytes": int(live_b + pb),
           "fwd_tensors_plus_plan_bytes": int(fwd_sum), "fwdbwd_tensors_plus_plan_bytes": int(bwd_sum),
           "free_bytes_change_fwd": int(free0) - int(free_f),
           "free_bytes_change_bwd": int(free1) - int(free2),
           "standard_attention_activation_model_bytes": activation_model_bytes(1, T, Hq, d)}
    del q, k, v, o, lse, fws, do, dq, dk, dv, ws, plan
    return rec


def run_memory(args, torch, mad):
    """Peak device memory of the path (LongCA-bench appendix A.4.2) for GLOBAL_SLIDING MHA (the pages'
    plotted case) and CAUSAL GQA from 1K to 48K, beside the pages' activation model of standard
    attention."""
    for mask, Hq, Hkv in [("GLOBAL_SLIDING", 64, 64), ("CAUSAL", 64, 8)]:
        for T in [1024, 2048, 4096, 8192, 16384, 32768, 49152]:
            d = 128
            kw = {"global_len": 256, "window": 2048} if mask == "GLOBAL_SLIDING" else {}
            rec = peak_memory_case(torch, mad, mask, T, Hq, Hkv, d, args.seed, kw)
            rec = {"workload": f"peak memory {mask} {'MHA' if Hq == Hkv else 'GQA'} {Hq}:{Hkv} T={T} d={d}",
                   "seq_len": T, "mask": mask, "heads_q": Hq, "heads_kv": Hkv, "head_dim": d, **rec,
                   "note": "peaks count every live tensor of the call (inputs, outputs, workspace) plus the plan"}
            print(json.dumps(rec), flush=True)


def mfma_sustained(torch, mad, n_wg=2048, iters=2048):
    """TFLOP/s of mad_probe_mfma: 4 * iters bf16 32x32x16 MFMAs per wave, 4 waves per workgroup."""
    sink = torch.empty(n_wg, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    L = mad.lib()
    for _ in range(2):
        mad._check(L.mad_probe_mfma(n_wg, iters, sink.data_ptr(), s.cuda_stream))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(s)
    reps = 5
    for _ in range(reps):
        mad._check(L.mad_probe_mfma(n_wg, iters, sink.data_ptr(), s.cuda_stream))
    ev[1].record(s)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    flop = float(n_wg) * 4 * 4 * iters * 32768.0
    return flop / (ms * 1e-3) / 1e12


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "detail": "no collectives or sharding are built: the kernels run one GPU's share (whole heads or one ring step) and value is that GPU's throughput"}))
        sys.exit(2)
    import torch
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": 3}))
        return
    import mask_aware_dense_amd as mad
    from oracle import masks as M

    torch.cuda.set_device(torch.device("cuda", 0))
    if args.suite:
        run_suite(args, torch, mad)
        return
    if args.memory:
        run_memory(args, torch, mad)
        return

    T, Hq, Hkv, d = args.seq, args.hq, args.hkv, args.d
    slices = mad.mask_slices(args.mask, T)
    t0 = time.perf_counter()
    plan = mad.mask_compile(slices, T, T)
    compile_s = time.perf_counter() - t0
    plan.upload()
    pairs = int(plan.stats(0)["pairs"][0]) * Hq
    flop_fwd = 4.0 * d * pairs
    flop_bwd = 10.0 * d * pairs

    r = Runner(torch, mad, plan, T, T, Hq, Hkv, d, args.seed)
    # the pages' protocol for a single-sequence mask: two runs of warm-up + timed steps, the median
    # reported (appendix A.4); each run times exactly `steps` steps between synchronisations
    runs = [r.time(args.steps, args.warmup, args.fwd_only) for _ in range(max(1, args.runs))]
    walls = [x[0] for x in runs]
    wall = float(np.median(walls))
    kern_ms = {n: float(np.mean([x[1][n] for x in runs])) for n in runs[0][1]}
    kern_med = {n: float(np.median([x[2][n] for x in runs])) for n in runs[0][2]}
    ms_step = wall * 1e3 / args.steps
    fwd_tflops = flop_fwd / (kern_ms["fwd"] * 1e-3) / 1e12
    run_vals = [(flop_fwd if args.fwd_only else flop_fwd + flop_bwd) * args.steps / w / 1e12 for w in walls]
    value = fwd_tflops if args.fwd_only else float(np.median(run_vals))
    workload = (f"{args.mask} attention {'fwd' if args.fwd_only else 'fwd+bwd'}, packed batch 1, "
                f"T={T}, GQA {Hq}:{Hkv}, head_dim {d}")

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "mask": args.mask, "seq_len": T, "heads_q": Hq, "heads_kv": Hkv,
                   "head_dim": d, "parallelism": "single GPU"},
        "fwd_tflops": fwd_tflops,
        "fwd_frac_peak": fwd_tflops / PEAK_BF16_TFLOPS,
        "fwdbwd_frac_peak": value / PEAK_BF16_TFLOPS,
        "kernel_ms_mean": kern_ms,
        "kernel_ms_median": kern_med,
        "runs": {"n": len(runs), "values": run_vals, "ms_per_step": [w * 1e3 / args.steps for w in walls],
                 "reported": "median"},
        "unmasked_pairs": pairs,
        "mask_compile_s": compile_s,
        "roofline": roofline(kern_ms, pairs, d, T, Hq, workload),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.fwd_only:
        # the matrix cores' sustained rate at the clock they hold under load (an MFMA-only
        # kernel), after the timed region: the ceiling the dominant kernel is compared with
        sus = mfma_sustained(torch, mad)
        out["mfma_sustained_tflops"] = sus
        out["roofline"]["frac_of_sustained"] = out["roofline"]["achieved"] / sus if sus else None
    if not args.no_cpu_baseline:
        q, k, v, do = r.host
        out["cpu_baseline"] = cpu_baseline(args, q, k, v, do, M.MaskSpec(args.mask, T, T), 1.0 / np.sqrt(d))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
