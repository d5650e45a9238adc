"""Python binding of libmad.so, the MI355X mask-aware attention library.

Argument marshalling only: every function here converts Python / numpy /
torch arguments to the C ABI declared in include/mad.h and calls it.  Mask
generation, mask compilation and every attention step run in the library
(host C++ and gfx950 HIP kernels).  PyTorch supplies device memory and the
current HIP stream.  Importing this module never falls back to another
implementation: if libmad.so is missing the import of the library raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "MadError", "lib", "Plan", "mask_slices", "ring_step_slices", "varlen_slices", "block_topk", "sparse_plan_device",
    "mask_compile", "sparse_plan", "attn_fwd", "attn_bwd", "attn_bwd_phases", "bwd_workspace_bytes", "bwd_kv_splits",
    "attn_bwd_static", "STATIC_WORKSPACE_BYTES",
    "block_mask", "block_mask_workspace_bytes", "lse_merge", "Ring", "BWD_DELTA", "BWD_DKDV", "BWD_DQ", "BWD_ALL",
    "PATTERNS", "SLICE_DTYPE",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmad.so")

PATTERNS = {
    "FULL": 0, "CAUSAL": 1, "SLIDING_WINDOW": 2, "FULL_DOCUMENT": 3, "CAUSAL_DOCUMENT": 4,
    "SLIDING_WINDOW_CAUSAL_DOCUMENT": 5, "PREFIX_LM": 6, "SHARED_QUESTION": 7,
    "GLOBAL_SLIDING": 8, "CAUSAL_BLOCKWISE": 9, "BLOCK_CAUSAL_DOCUMENT": 10,
    "PREFIX_LM_DOCUMENT": 11, "CAUSAL_BLOCKWISE_LAST": 12, "BLOCK_CAUSAL_DOCUMENT_GLOBAL": 13,
}

BWD_DELTA, BWD_DKDV, BWD_DQ, BWD_ALL = 1, 2, 4, 7

SLICE_DTYPE = np.dtype([("q0", "<i4"), ("q1", "<i4"), ("k0", "<i4"), ("k1", "<i4"),
                        ("type", "<i4"), ("window", "<i4")])


class MadError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"mad status {status}: {msg}")
        self.status = status


class _Slice(ctypes.Structure):
    _fields_ = [("q0", ctypes.c_int32), ("q1", ctypes.c_int32), ("k0", ctypes.c_int32),
                ("k1", ctypes.c_int32), ("type", ctypes.c_int32), ("window", ctypes.c_int32)]


class _Params(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("prefix", ctypes.c_int32), ("question", ctypes.c_int32),
                ("n_answers", ctypes.c_int32), ("global_len", ctypes.c_int32), ("block", ctypes.c_int32),
                ("doc_lens", ctypes.POINTER(ctypes.c_int32)), ("n_docs", ctypes.c_int32)]


_I32, _I64, _F32, _VP = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
_PI64 = ctypes.POINTER(ctypes.c_int64)
_PI32 = ctypes.POINTER(ctypes.c_int32)

_SIGS = {
    "mad_mask_slices": (_I32, [_I32, _I32, ctypes.POINTER(_Params), _VP, _I64, _PI64]),
    "mad_ring_step_slices": (_I32, [_I32, _I32, _I32, _I32, _I32, _VP, _I64, _PI64]),
    "mad_varlen_slices": (_I32, [_VP, _VP, _I32, _I32, _I32, _I32, _VP, _I64, _PI64]),
    "mad_block_topk": (_I32, [_VP, _I32, _I32, _I32, _I32, _VP]),
    "mad_mask_compile": (_I32, [_VP, _I64, _I32, _I32, ctypes.POINTER(_VP)]),
    "mad_sparse_plan": (_I32, [_I32, _VP, _I32, _VP, _I32, _VP, ctypes.POINTER(_VP)]),
    "mad_sparse_plan_device": (_I32, [_I32, _VP, _I32, _VP, _I32, _VP, _VP, ctypes.POINTER(_VP)]),
    "mad_plan_lists": (_I32, [_VP, _I32, _PI64, _PI64, _PI64, _VP, _VP, _VP, _VP]),
    "mad_probe_mfma": (_I32, [_I32, _I32, _VP, _VP]),
    "mad_plan_upload": (_I32, [_VP, _VP]),
    "mad_plan_stats": (_I32, [_VP, _I32, _VP, _PI64, _PI64, _PI64]),
    "mad_plan_info": (_I32, [_VP, _I32, _PI32, _PI32, _PI32, _PI32, _PI32, _PI32, _PI32]),
    "mad_plan_export": (_I32, [_VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP]),
    "mad_plan_destroy": (None, [_VP]),
    "mad_plan_device_bytes": (_I32, [_VP, ctypes.POINTER(ctypes.c_size_t)]),
    "mad_attn_fwd": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP, _F32, _VP,
                            ctypes.c_size_t, _VP]),
    "mad_bwd_workspace_bytes": (_I32, [_VP, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "mad_bwd_kv_splits": (_I32, [_VP, _I32, _I32, _PI32]),
    "mad_attn_bwd": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t,
                            _I32, _I32, _I32, _I32, _I32, _VP, _F32, _VP]),
    "mad_attn_bwd_phases": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t,
                                   _I32, _I32, _I32, _I32, _I32, _VP, _F32, ctypes.c_uint32, _VP]),
    "mad_attn_bwd_static": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                   _I32, _I32, _I32, _I32, _I32, _VP, _F32, _VP]),
    "mad_block_mask_workspace_bytes": (_I32, [_I32, _I32, _I32, _I32, _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "mad_block_mask": (_I32, [_VP, _VP, _I32, _I32, _I32, _I32, _I32, _I32, _VP, _I32, _VP, _I32, _I32, _F32,
                              _VP, ctypes.c_size_t, _VP, _VP, _VP]),
    "mad_lse_merge": (_I32, [_I32, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _VP]),
    "mad_ring_create": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(_VP)]),
    "mad_ring_info": (_I32, [_VP, _PI32, _PI64, ctypes.POINTER(ctypes.c_size_t)]),
    "mad_ring_fwd": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _F32, _VP]),
    "mad_ring_bwd": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _F32, _VP]),
    "mad_ring_destroy": (None, [_VP]),
    "mad_last_error": (ctypes.c_char_p, []),
    "mad_version": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmad.so (built in-tree by mask_aware_dense_amd.build); raise if absent."""
    global _lib
    if _lib is None:
        # torch first: its HIP runtime (libamdhip64.so.7) is then the one
        # libmad.so binds to, so both share one runtime and one device context
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not found: build it with `python -m mask_aware_dense_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise MadError(status, lib().mad_last_error().decode())


def _ptr(a) -> int:
    """Address of a numpy array's data, or of a torch tensor's storage."""
    if a is None:
        return None
    if hasattr(a, "data_ptr"):
        return a.data_ptr()
    return a.ctypes.data


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# --------------------------------------------------------------------------- masks

def mask_slices(pattern, T: int, window: int = 4096, prefix: int = -1, question: int = 2048,
                n_answers: int = 4, global_len: int = 256, block: int = 1024, doc_lens=None,
                answer_lens=None) -> np.ndarray:
    """Slices (structured array of SLICE_DTYPE) of a static pattern over a T x T mask.

    answer_lens (SHARED_QUESTION only) gives the answers' lengths instead of the equal split; the
    C ABI takes them in the doc_lens field."""
    pid = PATTERNS[pattern] if isinstance(pattern, str) else int(pattern)
    if answer_lens is not None:
        if doc_lens is not None:
            raise ValueError("give doc_lens or answer_lens, not both")
        doc_lens = answer_lens
    docs = np.ascontiguousarray(np.asarray([] if doc_lens is None else doc_lens, dtype=np.int32))
    prm = _Params(window, prefix, question, n_answers, global_len, block,
                  docs.ctypes.data_as(_PI32) if docs.size else None, docs.size)
    n = ctypes.c_int64(0)
    _check(lib().mad_mask_slices(pid, T, ctypes.byref(prm), None, 0, ctypes.byref(n)))
    out = np.zeros(n.value, dtype=SLICE_DTYPE)
    _check(lib().mad_mask_slices(pid, T, ctypes.byref(prm), out.ctypes.data if n.value else None,
                                 n.value, ctypes.byref(n)))
    return out


def varlen_slices(cu_q, cu_k=None, causal: bool = True, window: int = 0, bottom_right: bool = False) -> np.ndarray:
    """Slices of a batch of packed variable-length sequences from cumulative offsets (cu_seqlens).

    cu_k defaults to cu_q (self-attention).  Compile with Tq = cu_q[-1], Tk = cu_k[-1]."""
    cq = np.ascontiguousarray(np.asarray(cu_q, dtype=np.int32))
    ck = cq if cu_k is None else np.ascontiguousarray(np.asarray(cu_k, dtype=np.int32))
    if cq.ndim != 1 or ck.shape != cq.shape or cq.size == 0:
        raise ValueError("cu_q and cu_k must be 1-D with the same length >= 1")
    batch = cq.size - 1
    n = ctypes.c_int64(0)
    args = (cq.ctypes.data, ck.ctypes.data, batch, int(bool(causal)), int(window), int(bool(bottom_right)))
    _check(lib().mad_varlen_slices(*args, None, 0, ctypes.byref(n)))
    out = np.zeros(n.value, dtype=SLICE_DTYPE)
    _check(lib().mad_varlen_slices(*args, out.ctypes.data if n.value else None, n.value, ctypes.byref(n)))
    return out


def ring_step_slices(layout, n_ranks: int, chunk: int, rank: int, source: int) -> np.ndarray:
    """Slices of one ring step (layout "contiguous" or "headtail") in local coordinates."""
    lid = {"contiguous": 0, "headtail": 1}[layout] if isinstance(layout, str) else int(layout)
    n = ctypes.c_int64(0)
    _check(lib().mad_ring_step_slices(lid, n_ranks, chunk, rank, source, None, 0, ctypes.byref(n)))
    out = np.zeros(n.value, dtype=SLICE_DTYPE)
    _check(lib().mad_ring_step_slices(lid, n_ranks, chunk, rank, source,
                                      out.ctypes.data if n.value else None, n.value, ctypes.byref(n)))
    return out


def block_topk(scores: np.ndarray, sparsity_pct: int) -> np.ndarray:
    """Keep bitmap uint64 [G, n_qb, ceil(n_kb/64)] of the top-k key blocks per query block."""
    s = np.ascontiguousarray(scores, dtype=np.float32)
    G, nq, nk = s.shape
    keep = np.zeros((G, nq, (nk + 63) // 64), dtype=np.uint64)
    _check(lib().mad_block_topk(s.ctypes.data, G, nq, nk, int(sparsity_pct), keep.ctypes.data))
    return keep


class Plan:
    """Owner of a compiled mask (mad_plan*)."""

    def __init__(self, handle):
        self.handle = handle

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.mad_plan_destroy(h)

    def upload(self, stream=None) -> "Plan":
        _check(lib().mad_plan_upload(self.handle, _stream(stream)))
        return self

    def device_bytes(self) -> int:
        n = ctypes.c_size_t(0)
        _check(lib().mad_plan_device_bytes(self.handle, ctypes.byref(n)))
        return n.value

    def info(self, which: int = 0) -> dict:
        v = [ctypes.c_int32() for _ in range(7)]
        _check(lib().mad_plan_info(self.handle, which, *[ctypes.byref(x) for x in v]))
        return dict(zip(("Tq", "Tk", "n_groups", "BM", "BN", "n_qt", "n_kt"), (x.value for x in v)))

    def stats(self, which: int = 0) -> dict:
        G = self.info(which)["n_groups"]
        pairs = np.zeros(G, dtype=np.int64)
        f, p, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().mad_plan_stats(self.handle, which, pairs.ctypes.data, ctypes.byref(f),
                                    ctypes.byref(p), ctypes.byref(e)))
        return {"pairs": pairs, "full": f.value, "partial": p.value, "empty": e.value}

    def export(self, which: int = 0, group: int = 0) -> dict:
        inf = self.info(which)
        nq, nk = inf["n_qt"], inf["n_kt"]
        cls = np.zeros(nq * nk, dtype=np.uint8)
        csr_ptr = np.zeros(nq + 1, dtype=np.int64)
        csc_ptr = np.zeros(nk + 1, dtype=np.int64)
        _check(lib().mad_plan_export(self.handle, which, group, cls.ctypes.data, csr_ptr.ctypes.data,
                                     None, csc_ptr.ctypes.data, None))
        csr_idx = np.zeros(max(int(csr_ptr[-1]), 1), dtype=np.int32)
        csc_idx = np.zeros(max(int(csc_ptr[-1]), 1), dtype=np.int32)
        _check(lib().mad_plan_export(self.handle, which, group, None, None, csr_idx.ctypes.data,
                                     None, csc_idx.ctypes.data))
        return {"classes": cls.reshape(nq, nk), "csr_ptr": csr_ptr, "csr_idx": csr_idx[:csr_ptr[-1]],
                "csc_ptr": csc_ptr, "csc_idx": csc_idx[:csc_ptr[-1]]}

    def lists(self, which: int = 0) -> dict:
        """Raw visit lists of tiling `which` as the kernels read them (ptr, ent, ent_aux, order)."""
        n = [ctypes.c_int64(0) for _ in range(3)]
        _check(lib().mad_plan_lists(self.handle, which, *(ctypes.byref(x) for x in n), None, None, None, None))
        ptr, ent, aux, order = (np.zeros(max(int(x.value), 1), dtype=np.int32) for x in (n[0], n[1], n[1], n[2]))
        _check(lib().mad_plan_lists(self.handle, which, None, None, None, ptr.ctypes.data, ent.ctypes.data,
                                    aux.ctypes.data, order.ctypes.data))
        return {"ptr": ptr[:n[0].value], "ent": ent[:n[1].value], "ent_aux": aux[:n[1].value],
                "order": order[:n[2].value]}


def mask_compile(slices: np.ndarray, Tq: int, Tk: int) -> Plan:
    s = np.ascontiguousarray(slices, dtype=SLICE_DTYPE)
    h = ctypes.c_void_p()
    _check(lib().mad_mask_compile(s.ctypes.data if s.size else None, s.size, Tq, Tk, ctypes.byref(h)))
    return Plan(h.value)


def sparse_plan(n_groups: int, q_edges, k_edges, keep: np.ndarray) -> Plan:
    qe = np.ascontiguousarray(q_edges, dtype=np.int32)
    ke = np.ascontiguousarray(k_edges, dtype=np.int32)
    kp = np.ascontiguousarray(keep, dtype=np.uint64)
    h = ctypes.c_void_p()
    _check(lib().mad_sparse_plan(n_groups, qe.ctypes.data, qe.size - 1, ke.ctypes.data, ke.size - 1,
                                 kp.ctypes.data, ctypes.byref(h)))
    return Plan(h.value)


def sparse_plan_device(n_groups: int, q_edges, k_edges, keep, stream=None) -> Plan:
    """Block-sparse plan compiled on the GPU from a device keep bitmap (torch uint64 tensor
    [G, n_qb, ceil(n_kb/64)], e.g. block_mask's output); edges are host arrays."""
    qe = np.ascontiguousarray(q_edges, dtype=np.int32)
    ke = np.ascontiguousarray(k_edges, dtype=np.int32)
    h = ctypes.c_void_p()
    _check(lib().mad_sparse_plan_device(n_groups, qe.ctypes.data, qe.size - 1, ke.ctypes.data, ke.size - 1,
                                        _ptr(keep), _stream(stream), ctypes.byref(h)))
    return Plan(h.value)


# --------------------------------------------------------------------------- attention

def _qkv_strides(q, k, v):
    arr = (ctypes.c_int64 * 6)(q.stride(0), q.stride(1), k.stride(0), k.stride(1), v.stride(0), v.stride(1))
    for t in (q, k, v):
        if t.stride(2) != 1:
            raise MadError(2, "head dimension must be contiguous")
    return arr


def _check_tensors(q, k, v, packed, lse):
    """Argument checks the C ABI cannot make from raw pointers: dtypes, exact shapes, one device, and
    packed (contiguous) layouts for every tensor the kernels address as packed.  q / k / v may be
    strided views (their strides are passed on); `packed` maps names to (tensor, shape) pairs."""
    import torch
    if len(q.shape) != 3 or len(k.shape) != 3 or len(v.shape) != 3:
        raise MadError(1, "q, k, v must be 3-D [tokens, heads, head_dim]")
    if tuple(v.shape) != tuple(k.shape):
        raise MadError(1, f"v shape {tuple(v.shape)} differs from k shape {tuple(k.shape)}")
    if q.shape[2] != k.shape[2]:
        raise MadError(1, "q and k head dims differ")
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16:
            raise MadError(1, f"{name} must be bfloat16, got {t.dtype}")
        if t.device != dev:
            raise MadError(1, f"{name} is on {t.device}, q on {dev}")
    for name, (t, shape) in packed.items():
        if t is None:
            raise MadError(1, f"{name} must not be None")
        if tuple(t.shape) != tuple(shape):
            raise MadError(1, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if t.dtype != torch.bfloat16:
            raise MadError(1, f"{name} must be bfloat16, got {t.dtype}")
        if t.device != dev:
            raise MadError(1, f"{name} is on {t.device}, q on {dev}")
        if not t.is_contiguous():
            raise MadError(1, f"{name} must be contiguous (packed [tokens, heads, head_dim])")
    if lse is not None:
        Hq, Tq = q.shape[1], q.shape[0]
        if tuple(lse.shape) != (Hq, Tq):
            raise MadError(1, f"lse must have shape {(Hq, Tq)}, got {tuple(lse.shape)}")
        if lse.dtype != torch.float32:
            raise MadError(1, f"lse must be float32, got {lse.dtype}")
        if lse.device != dev:
            raise MadError(1, f"lse is on {lse.device}, q on {dev}")
        if not lse.is_contiguous():
            raise MadError(1, "lse must be contiguous [heads, tokens]")
    if dev.type != "cuda":
        raise MadError(1, f"tensors must be on a GPU, got {dev}")
    if dev.index is not None and torch.cuda.is_available() and dev.index != torch.cuda.current_device():
        raise MadError(1, f"tensors are on {dev} but the current device is cuda:{torch.cuda.current_device()}")


def _check_workspace(workspace):
    if workspace is None:
        return 0
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise MadError(1, "workspace must be a contiguous GPU tensor")
    return workspace.numel() * workspace.element_size()


FWD_WORKSPACE_BYTES = 256


def attn_fwd(plan: Plan, q, k, v, o, lse, scale: float, stream=None, workspace=None):
    """Forward into preallocated o [Tq,Hq,d] bf16 and lse [Hq,Tq] fp32 (torch CUDA tensors).  workspace:
    None, or a device buffer of at least FWD_WORKSPACE_BYTES (its work-item counters; not shared by calls
    that may run at the same time)."""
    Tq, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    _check_tensors(q, k, v, {"o": (o, (Tq, Hq, d))}, lse)
    st = _qkv_strides(q, k, v)
    nbytes = _check_workspace(workspace)
    _check(lib().mad_attn_fwd(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), Tq, Tk, Hq, Hkv, d,
                              st, float(scale), _ptr(workspace), nbytes, _stream(stream)))


def bwd_workspace_bytes(plan: Plan, Tq: int, Tk: int, Hq: int, Hkv: int, d: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().mad_bwd_workspace_bytes(plan.handle, Tq, Tk, Hq, Hkv, d, ctypes.byref(n)))
    return n.value


def bwd_kv_splits(plan: Plan, Hq: int, Hkv: int) -> int:
    """Workgroups per key-tile column of the backward's dK/dV kernel (1: no cut columns)."""
    n = ctypes.c_int32()
    _check(lib().mad_bwd_kv_splits(plan.handle, Hq, Hkv, ctypes.byref(n)))
    return n.value


def attn_bwd(plan: Plan, q, k, v, o, d_o, lse, dq, dk, dv, workspace, scale: float, stream=None):
    """Backward into preallocated dq, dk, dv; workspace is a device buffer (uint8 tensor)."""
    Tq, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    _check_tensors(q, k, v, {"o": (o, (Tq, Hq, d)), "d_o": (d_o, (Tq, Hq, d)), "dq": (dq, (Tq, Hq, d)),
                             "dk": (dk, (Tk, Hkv, d)), "dv": (dv, (Tk, Hkv, d))}, lse)
    st = _qkv_strides(q, k, v)
    nbytes = _check_workspace(workspace)
    _check(lib().mad_attn_bwd(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse),
                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), nbytes, Tq, Tk, Hq, Hkv, d,
                              st, float(scale), _stream(stream)))


STATIC_WORKSPACE_BYTES = 64 << 20


def attn_bwd_static(plan: Plan, q, k, v, o, d_o, lse, dq, dk, dv, scale: float, stream=None):
    """Backward with the library's static device workspace (no workspace argument, no allocation)."""
    Tq, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    _check_tensors(q, k, v, {"o": (o, (Tq, Hq, d)), "d_o": (d_o, (Tq, Hq, d)), "dq": (dq, (Tq, Hq, d)),
                             "dk": (dk, (Tk, Hkv, d)), "dv": (dv, (Tk, Hkv, d))}, lse)
    st = _qkv_strides(q, k, v)
    _check(lib().mad_attn_bwd_static(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse),
                                     _ptr(dq), _ptr(dk), _ptr(dv), Tq, Tk, Hq, Hkv, d, st, float(scale),
                                     _stream(stream)))


def attn_bwd_phases(plan: Plan, q, k, v, o, d_o, lse, dq, dk, dv, workspace, scale: float, phases: int,
                    stream=None):
    """One or more of the backward's launches (BWD_DELTA, BWD_DKDV, BWD_DQ bit set)."""
    Tq, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    _check_tensors(q, k, v, {"o": (o, (Tq, Hq, d)), "d_o": (d_o, (Tq, Hq, d)), "dq": (dq, (Tq, Hq, d)),
                             "dk": (dk, (Tk, Hkv, d)), "dv": (dv, (Tk, Hkv, d))}, lse)
    st = _qkv_strides(q, k, v)
    nbytes = _check_workspace(workspace)
    _check(lib().mad_attn_bwd_phases(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse),
                                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), nbytes, Tq, Tk, Hq, Hkv, d,
                                     st, float(scale), int(phases), _stream(stream)))


# --------------------------------------------------------------------------- merge and ring

def lse_merge(o_parts, lse_parts, o, lse, stream=None):
    """Merge partial results (lists of bf16 [Tq, Hq, d] and fp32 [Hq, Tq] device tensors) into o, lse."""
    n = len(o_parts)
    if len(lse_parts) != n:
        raise ValueError("o_parts and lse_parts differ in length")
    Tq, Hq, d = o.shape
    op = (ctypes.c_void_p * max(n, 1))(*[_ptr(x) for x in o_parts])
    lp = (ctypes.c_void_p * max(n, 1))(*[_ptr(x) for x in lse_parts])
    _check(lib().mad_lse_merge(n, ctypes.cast(op, _VP), ctypes.cast(lp, _VP), _ptr(o), _ptr(lse), Tq, Hq, d,
                               _stream(stream)))


class Ring:
    """Owner of one rank's ring context-parallel share (mad_ring*)."""

    def __init__(self, layout, n_ranks: int, chunk: int, rank: int, Hq: int, Hkv: int, d: int):
        lid = {"contiguous": 0, "headtail": 1}[layout] if isinstance(layout, str) else int(layout)
        h = ctypes.c_void_p()
        _check(lib().mad_ring_create(lid, n_ranks, chunk, rank, Hq, Hkv, d, ctypes.byref(h)))
        self.handle = h.value

    def __del__(self):
        if getattr(self, "handle", None):
            lib().mad_ring_destroy(self.handle)
            self.handle = None

    def info(self) -> dict:
        n = ctypes.c_int32(0)
        p = ctypes.c_int64(0)
        b = ctypes.c_size_t(0)
        _check(lib().mad_ring_info(self.handle, ctypes.byref(n), ctypes.byref(p), ctypes.byref(b)))
        return {"n_steps": n.value, "pairs_per_head": p.value, "device_bytes": b.value}

    def fwd(self, q, k, v, o, lse, scale: float, stream=None):
        _check(lib().mad_ring_fwd(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), float(scale),
                                  _stream(stream)))

    def bwd(self, q, k, v, o, d_o, lse, dq, dk, dv, scale: float, stream=None):
        _check(lib().mad_ring_bwd(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse), _ptr(dq),
                                  _ptr(dk), _ptr(dv), float(scale), _stream(stream)))


# --------------------------------------------------------------------------- dynamic block masks

def block_mask_workspace_bytes(n_groups: int, Hkv: int, n_qb: int, n_kb: int, d: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mad_block_mask_workspace_bytes(n_groups, Hkv, n_qb, n_kb, d, ctypes.byref(n)))
    return n.value


def block_mask(q, k, n_groups: int, q_edges, k_edges, sparsity_pct: int, scale: float, keep, workspace,
               scores=None, stream=None):
    """Keep bitmap (device uint64 tensor [G, n_qb, ceil(n_kb/64)], written) of the top-k key blocks per
    query block by mean-pooled block scores; q_edges / k_edges are device int32 tensors."""
    Tq, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().mad_block_mask(_ptr(q), _ptr(k), Tq, Tk, Hq, Hkv, d, n_groups, _ptr(q_edges), q_edges.numel() - 1,
                                _ptr(k_edges), k_edges.numel() - 1, int(sparsity_pct), float(scale), _ptr(workspace),
                                nbytes, _ptr(keep), _ptr(scores), _stream(stream)))
