"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module draws random numbers and nothing else: it holds none of the
attention or mask arithmetic.  Every generator is a pure function of its seed
and sizes, so the GPU run and the CPU oracle can each call it and receive the
same values.

The pages measure on real corpora (Pile, ProLong); those are not used here.
Document lengths are drawn log-uniformly in [512, 16384] tokens and truncated
to fill the packed total, as in the dense-kernel workload description
(LongCA-bench, section 2.1.2 "Input data sampling").  Block-sparse inputs are
random block scores per (mask group, query block, key block), as in appendix
A.2 "Score calculation" (random scores isolate the kernel).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "qkv", "grad_out", "qkv_device", "grad_out_device", "doc_lengths", "block_scores", "variable_block_sizes",
    "answer_lengths",
]


def _torch():
    import torch  # imported lazily: the host-only tests do not need it
    return torch


def qkv(seed: int, Tq: int, Tk: int, Hq: int, Hkv: int, d: int):
    """Q [Tq,Hq,d], K [Tk,Hkv,d], V [Tk,Hkv,d] as CPU bf16 tensors.

    Each is N(0,1) drawn in fp32 from one CPU generator seeded with `seed`, in
    the order Q, K, V, then rounded to bf16 (round to nearest even).
    """
    torch = _torch()
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    q = torch.randn((Tq, Hq, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((Tk, Hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((Tk, Hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v


def grad_out(seed: int, Tq: int, Hq: int, d: int):
    """dO [Tq,Hq,d] CPU bf16, N(0,1) from its own stream (seed, tag 7)."""
    torch = _torch()
    g = torch.Generator(device="cpu").manual_seed(int(seed) * 1000003 + 7)
    return torch.randn((Tq, Hq, d), generator=g, dtype=torch.float32).to(torch.bfloat16)


def qkv_device(seed: int, Tq: int, Tk: int, Hq: int, Hkv: int, d: int, device="cuda"):
    """The same distribution drawn on the GPU (for the largest sizes, where the CPU generator
    would take minutes): N(0,1) fp32 from one device generator seeded with `seed`, in the order
    Q, K, V, rounded to bf16.  Deterministic for a seed on a given device type; the values
    differ from qkv's, so a test copies back what its oracle needs."""
    torch = _torch()
    g = torch.Generator(device=device).manual_seed(int(seed))
    q = torch.randn((Tq, Hq, d), generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
    k = torch.randn((Tk, Hkv, d), generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
    v = torch.randn((Tk, Hkv, d), generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
    return q, k, v


def grad_out_device(seed: int, Tq: int, Hq: int, d: int, device="cuda"):
    """dO [Tq,Hq,d] bf16 drawn on the GPU from its own stream (seed, tag 7)."""
    torch = _torch()
    g = torch.Generator(device=device).manual_seed(int(seed) * 1000003 + 7)
    return torch.randn((Tq, Hq, d), generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)


def doc_lengths(seed: int, T: int, lo: int = 512, hi: int = 16384) -> np.ndarray:
    """Packed document lengths summing exactly to T (int64).

    L = floor(exp(U(ln lo, ln hi))) drawn until the running sum reaches T; the
    last document is truncated so the lengths sum to T.
    """
    if T <= 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng([int(seed), 1])
    out = []
    total = 0
    while total < T:
        L = int(np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi)))))
        L = max(1, min(L, T - total))
        out.append(L)
        total += L
    return np.asarray(out, dtype=np.int64)


def block_scores(seed: int, n_groups: int, n_qb: int, n_kb: int) -> np.ndarray:
    """Random block importance scores, float32 [n_groups, n_qb, n_kb], U[0,1)."""
    rng = np.random.default_rng([int(seed), 2])
    return rng.random((n_groups, n_qb, n_kb), dtype=np.float32)


def variable_block_sizes(seed: int, T: int, lo: int = 32, hi: int = 256) -> np.ndarray:
    """Block sizes drawn from U{lo..hi} until they cover T; the last is truncated."""
    if T <= 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng([int(seed), 3])
    out = []
    total = 0
    while total < T:
        b = int(rng.integers(lo, hi + 1))
        b = min(b, T - total)
        out.append(b)
        total += b
    return np.asarray(out, dtype=np.int64)


def answer_lengths(seed: int, rest: int, n_answers: int) -> np.ndarray:
    """Answer lengths of a Shared Question mask (int64, n_answers entries summing to `rest`):
    n_answers - 1 cut points drawn uniformly from 0..rest and sorted."""
    rng = np.random.default_rng([int(seed), 4])
    cuts = np.sort(rng.integers(0, rest + 1, size=max(n_answers - 1, 0)))
    edges = np.concatenate([[0], cuts, [rest]]).astype(np.int64)
    return np.diff(edges)
