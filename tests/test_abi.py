"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments with the documented status codes before touching the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import mask_aware_dense_amd as mad

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "mad.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mad_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert "mad_attn_fwd" in names and "mad_attn_bwd" in names and "mad_mask_compile" in names
    L = mad.lib()
    for n in names:
        assert hasattr(L, n), n
    assert b"gfx950" in L.mad_version()


def _status(e):
    return e.value.status


def test_mask_slice_errors():
    with pytest.raises(mad.MadError) as e:
        mad.mask_slices(99, 10)
    assert _status(e) == 1
    with pytest.raises(mad.MadError) as e:
        mad.mask_slices("CAUSAL_DOCUMENT", 10, doc_lens=[3, 3])
    assert _status(e) == 1 and "sum" in str(e.value)
    with pytest.raises(mad.MadError):
        mad.mask_slices("SLIDING_WINDOW", 10, window=0)
    with pytest.raises(mad.MadError):
        mad.ring_step_slices("headtail", 4, 7, 0, 1)  # odd chunk
    with pytest.raises(mad.MadError):
        mad.ring_step_slices("contiguous", 4, 8, 4, 1)  # rank out of range
    with pytest.raises(mad.MadError):
        mad.block_topk(np.zeros((1, 2, 3), np.float32), 101)
    nan = np.zeros((1, 2, 3), np.float32)
    nan[0, 1, 2] = np.nan
    with pytest.raises(mad.MadError):
        mad.block_topk(nan, 50)


def test_compile_errors():
    bad = np.array([(0, 11, 0, 5, 0, 0)], dtype=mad.SLICE_DTYPE)
    with pytest.raises(mad.MadError) as e:
        mad.mask_compile(bad, 10, 10)
    assert _status(e) == 1 and "out of range" in str(e.value)
    bad = np.array([(0, 5, 0, 5, 2, 0)], dtype=mad.SLICE_DTYPE)
    with pytest.raises(mad.MadError):
        mad.mask_compile(bad, 10, 10)
    bad = np.array([(0, 5, 0, 5, 0, 3)], dtype=mad.SLICE_DTYPE)  # window on a FULL slice
    with pytest.raises(mad.MadError):
        mad.mask_compile(bad, 10, 10)
    with pytest.raises(mad.MadError):
        mad.sparse_plan(1, [0, 5, 5, 9], [0, 9], np.ones((1, 3, 1), np.uint64))
    with pytest.raises(mad.MadError):
        mad.sparse_plan(1, [1, 9], [0, 9], np.ones((1, 1, 1), np.uint64))


class _Fake:
    """Stand-in GPU tensor: shape, strides, dtype, device and a (never dereferenced) address."""

    def __init__(self, shape, addr=4096, dtype=None, device=None, contiguous=True):
        import torch
        self.shape = shape
        self._addr = addr
        st = [1] * len(shape)
        for i in range(len(shape) - 2, -1, -1):
            st[i] = st[i + 1] * shape[i + 1]
        self._st = st
        if dtype is None:
            dtype = torch.float32 if len(shape) == 2 else torch.bfloat16 if len(shape) == 3 else torch.uint8
        self.dtype = dtype
        self.device = torch.device("cuda", 0) if device is None else device
        self._contig = contiguous

    def stride(self, i):
        return self._st[i]

    def data_ptr(self):
        return self._addr

    def numel(self):
        return int(np.prod(self.shape))

    def element_size(self):
        return 1

    def is_contiguous(self):
        return self._contig


def test_attention_argument_errors_launch_nothing():
    """Every check below fails before any HIP call (no GPU in this container)."""
    T = 64
    plan = mad.mask_compile(mad.mask_slices("CAUSAL", T), T, T)
    q, k, v = _Fake((T, 4, 128)), _Fake((T, 2, 128)), _Fake((T, 2, 128))
    o, lse = _Fake((T, 4, 128)), _Fake((4, T))
    with pytest.raises(mad.MadError) as e:
        mad.attn_fwd(plan, _Fake((T, 4, 96)), _Fake((T, 2, 96)), _Fake((T, 2, 96)), _Fake((T, 4, 96)), lse, 0.1,
                     stream=0)
    assert _status(e) == 2  # head dim
    with pytest.raises(mad.MadError) as e:
        mad.attn_fwd(plan, _Fake((T, 3, 128)), k, v, _Fake((T, 3, 128)), _Fake((3, T)), 0.1, stream=0)
    assert _status(e) == 1  # Hq % Hkv
    with pytest.raises(mad.MadError) as e:
        mad.attn_fwd(plan, _Fake((T + 1, 4, 128)), k, v, _Fake((T + 1, 4, 128)), _Fake((4, T + 1)), 0.1, stream=0)
    assert _status(e) == 1 and "compiled for" in str(e.value)
    with pytest.raises(mad.MadError) as e:
        mad.attn_fwd(plan, q, k, v, o, lse, 0.1, stream=0)
    assert _status(e) == 1 and "not uploaded" in str(e.value)
    with pytest.raises(mad.MadError) as e:
        mad.attn_bwd(plan, q, k, v, o, q, lse, q, k, v, _Fake((16,)), 0.1, stream=0)
    assert _status(e) == 1
    with pytest.raises(mad.MadError) as e:
        mad.attn_bwd_phases(plan, q, k, v, o, q, lse, q, k, v, _Fake((1 << 20,)), 0.1, 8, stream=0)
    assert _status(e) == 1 and "phase" in str(e.value)
    assert mad.bwd_workspace_bytes(plan, T, T, 4, 2, 128) >= 4 * T * 4
    L = mad.lib()
    assert L.mad_attn_fwd(None, None, None, None, None, None, 1, 1, 1, 1, 64, None, ctypes.c_float(1.0), None, 0,
                          None) == 1
    assert b"plan is NULL" in L.mad_last_error()


def test_merge_and_ring_errors():
    """Argument checks of the LSE merge and the ring object fail before any device work."""
    L = mad.lib()
    null = ctypes.c_void_p(0)
    arr = (ctypes.c_void_p * 1)(0)
    # n_parts out of range, bad head dim, NULL part arrays
    assert L.mad_lse_merge(0, arr, arr, null, null, 4, 2, 128, null) == 1
    assert L.mad_lse_merge(33, arr, arr, null, null, 4, 2, 128, null) == 1
    assert L.mad_lse_merge(1, arr, arr, null, null, 4, 2, 96, null) == 2
    assert L.mad_lse_merge(1, null, null, null, null, 4, 2, 128, null) == 1
    assert L.mad_lse_merge(1, arr, arr, null, null, 4, 0, 128, null) == 1
    # a NULL part pointer with a real output
    assert L.mad_lse_merge(1, arr, arr, ctypes.c_void_p(256), ctypes.c_void_p(256), 4, 2, 128, null) == 1
    assert b"part" in L.mad_last_error()
    h = ctypes.c_void_p()
    for args, st in [((2, 4, 64, 0, 4, 2, 128), 1),   # layout
                     ((0, 0, 64, 0, 4, 2, 128), 1),   # n_ranks
                     ((0, 33, 64, 0, 4, 2, 128), 1),
                     ((1, 4, 63, 0, 4, 2, 128), 1),   # odd head-tail chunk
                     ((0, 4, 64, 4, 4, 2, 128), 1),   # rank
                     ((0, 4, 64, 0, 4, 3, 128), 1),   # Hq % Hkv
                     ((0, 4, 64, 0, 4, 2, 80), 2)]:   # head dim
        assert L.mad_ring_create(*args, ctypes.byref(h)) == st, args
    assert L.mad_ring_create(0, 4, 64, 0, 4, 2, 128, None) == 1
    assert L.mad_ring_info(None, None, None, None) == 1
    assert L.mad_ring_fwd(None, null, null, null, null, null, 1.0, null) == 1
    assert L.mad_ring_bwd(None, null, null, null, null, null, null, null, null, null, 1.0, null) == 1
    L.mad_ring_destroy(None)


def test_block_mask_errors():
    """Argument checks of the GPU block-mask generator fail before any device work."""
    L = mad.lib()
    n = ctypes.c_size_t(0)
    assert L.mad_block_mask_workspace_bytes(8, 8, 16, 16, 128, ctypes.byref(n)) == 0
    assert n.value == 8 * 16 * 128 * 4 + 8 * 16 * 128 * 4
    assert L.mad_block_mask_workspace_bytes(8, 8, 16, 16, 96, ctypes.byref(n)) == 2
    assert L.mad_block_mask_workspace_bytes(0, 8, 16, 16, 128, ctypes.byref(n)) == 1
    p = ctypes.c_void_p(4096)
    base = (p, p, 1024, 1024, 8, 2, 128)
    def call(*over, groups=2, nqb=8, nkb=8, pct=50, ws=1 << 20, **kw):
        args = list(base)
        for i, v in over:
            args[i] = v
        return L.mad_block_mask(*args, groups, p, nqb, p, nkb, pct, ctypes.c_float(0.1), p, ws, p, None, None)
    assert call(groups=3) == 1        # does not divide Hq
    assert call(groups=1) == 1        # group spans two KV heads
    assert call((6, 80)) == 2         # head dim
    assert call(pct=101) == 1
    assert call(nkb=9000) == 1        # more blocks than keys
    assert call(nqb=0) == 1
    assert call(ws=16) == 1           # workspace too small
    assert L.mad_block_mask(None, p, 1024, 1024, 8, 2, 128, 2, p, 8, p, 8, 50, ctypes.c_float(0.1), p, 1 << 20,
                            p, None, None) == 1


def test_sparse_plan_device_errors():
    """Argument checks of the GPU plan compiler fail before any device work."""
    L = mad.lib()
    qe = np.array([0, 64, 128], dtype=np.int32)
    ke = np.array([0, 64, 100], dtype=np.int32)
    bad = np.array([0, 64, 64], dtype=np.int32)
    keep = ctypes.c_void_p(4096)
    out = ctypes.c_void_p()

    def call(G=2, q=qe, nqb=2, k=ke, nkb=2, kp=keep, o=ctypes.byref(out)):
        return L.mad_sparse_plan_device(G, q.ctypes.data if q is not None else None, nqb,
                                        k.ctypes.data if k is not None else None, nkb, kp, None, o)

    assert call(o=None) == 1
    assert call(kp=None) == 1
    assert call(q=None) == 1
    assert call(G=0) == 1
    assert call(nkb=0) == 1
    assert call(k=bad) == 1                      # not strictly increasing
    assert call(q=np.array([1, 64, 128], dtype=np.int32)) == 1  # does not start at 0
    assert call(kp=ctypes.c_void_p(4100)) == 1   # keep not 8-byte aligned
    assert out.value is None


def test_plan_lists_host_plan():
    """Raw lists of a host-compiled plan agree with its export (CSR for tiling 0, CSC for tiling 1)."""
    T = 700
    plan = mad.mask_compile(mad.mask_slices("CAUSAL", T), T, T)
    for w in (0, 1):
        li = plan.lists(w)
        ex = plan.export(w, 0)
        ptr = ex["csr_ptr"] if w == 0 else ex["csc_ptr"]
        idx = ex["csr_idx"] if w == 0 else ex["csc_idx"]
        assert np.array_equal(li["ptr"], ptr)
        assert np.array_equal(li["ent"] & 0x7fffffff, idx)
        assert sorted(li["order"].tolist()) == list(range(len(ptr) - 1))


def test_probe_mfma_errors():
    L = mad.lib()
    assert L.mad_probe_mfma(0, 10, ctypes.c_void_p(4096), None) == 1
    assert L.mad_probe_mfma(4, 0, ctypes.c_void_p(4096), None) == 1
    assert L.mad_probe_mfma(4, 10, None, None) == 1


def test_binding_rejects_mismatched_tensors():
    """The binding checks dtypes, exact shapes, one device and packed layouts before calling the
    library: the kernels address o, d_o, dq, dk, dv and lse as packed tensors."""
    import torch
    T, Hq, Hkv, d = 64, 4, 2, 128
    plan = mad.mask_compile(mad.mask_slices("CAUSAL", T), T, T)
    q, k, v = _Fake((T, Hq, d)), _Fake((T, Hkv, d)), _Fake((T, Hkv, d))
    o, lse = _Fake((T, Hq, d)), _Fake((Hq, T))
    ws = _Fake((1 << 16,))

    def fwd(**over):
        a = dict(q=q, k=k, v=v, o=o, lse=lse)
        a.update(over)
        with pytest.raises(mad.MadError) as e:
            mad.attn_fwd(plan, a["q"], a["k"], a["v"], a["o"], a["lse"], 0.1, stream=0)
        return str(e.value)

    def bwd(**over):
        a = dict(q=q, k=k, v=v, o=o, d_o=_Fake((T, Hq, d)), lse=lse, dq=_Fake((T, Hq, d)), dk=_Fake((T, Hkv, d)),
                 dv=_Fake((T, Hkv, d)), ws=ws)
        a.update(over)
        with pytest.raises(mad.MadError) as e:
            mad.attn_bwd(plan, a["q"], a["k"], a["v"], a["o"], a["d_o"], a["lse"], a["dq"], a["dk"], a["dv"], a["ws"],
                         0.1, stream=0)
        return str(e.value)

    assert "q must be bfloat16" in fwd(q=_Fake((T, Hq, d), dtype=torch.float32))
    assert "v shape" in fwd(v=_Fake((T, 1, d)))
    assert "o must have shape" in fwd(o=_Fake((T - 1, Hq, d)))
    assert "o must be bfloat16" in fwd(o=_Fake((T, Hq, d), dtype=torch.float16))
    assert "o must be contiguous" in fwd(o=_Fake((T, Hq, d), contiguous=False))
    assert "lse must have shape" in fwd(lse=_Fake((T, Hq)))
    assert "lse must be float32" in fwd(lse=_Fake((Hq, T), dtype=torch.bfloat16))
    assert "is on cpu" in fwd(o=_Fake((T, Hq, d), device=torch.device("cpu")))
    assert "k is on cuda:1" in fwd(k=_Fake((T, Hkv, d), device=torch.device("cuda", 1)))
    assert "dk must have shape" in bwd(dk=_Fake((T, Hq, d)))
    assert "dv must be contiguous" in bwd(dv=_Fake((T, Hkv, d), contiguous=False))
    assert "d_o must be bfloat16" in bwd(d_o=_Fake((T, Hq, d), dtype=torch.float32))
    assert "dq must not be None" in bwd(dq=None)
    assert "workspace must be a contiguous GPU tensor" in bwd(ws=_Fake((256,), device=torch.device("cpu")))
    # a correct call still reaches the library's own checks (the plan is not uploaded)
    assert "not uploaded" in bwd()
