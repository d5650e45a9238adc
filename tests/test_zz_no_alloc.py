"""The allocation-free backward (mad_attn_bwd_static, the library's static device workspace) against
the backward with a caller workspace (mad_attn_bwd), through the C ABI: two calls in a row, the
second on a smaller input, each checked to the parity bar against the workspace form; and a call
needing more than the static workspace is refused before anything is launched."""
import ctypes

import numpy as np
import pytest

import _gpu
from mad_inputs import grad_out, qkv

pytestmark = pytest.mark.gpu


def _case(pattern, T, Hq, Hkv, d, seed):
    import torch
    import mask_aware_dense_amd as mad
    dev = torch.device("cuda", 0)
    plan = mad.mask_compile(mad.mask_slices(pattern, T, global_len=64, window=512), T, T).upload()
    q, k, v = (x.to(dev) for x in qkv(seed, T, T, Hq, Hkv, d))
    do = grad_out(seed, T, Hq, d).to(dev)
    scale = 1.0 / np.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    mad.attn_fwd(plan, q, k, v, o, lse, scale)
    ref = [torch.empty_like(x) for x in (q, k, v)]
    ws = torch.empty(mad.bwd_workspace_bytes(plan, T, T, Hq, Hkv, d), dtype=torch.uint8, device=dev)
    mad.attn_bwd(plan, q, k, v, o, do, lse, *ref, ws, scale)
    got = [torch.full_like(x, float("nan")) for x in (q, k, v)]
    mad.attn_bwd_static(plan, q, k, v, o, do, lse, *got, scale)
    torch.cuda.synchronize()
    splits = mad.bwd_kv_splits(plan, Hq, Hkv)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        a64, b64 = a.float().cpu().numpy().astype(np.float64), b.float().cpu().numpy().astype(np.float64)
        _gpu.check_close(name, a64, b64, _gpu.TOL_BWD)
        if splits == 1:  # one workgroup per dK/dV column: the two forms run the same kernels bit for bit
            assert np.array_equal(a64, b64), name
    return splits


def test_static_workspace_two_calls_second_smaller():
    print("case static workspace: GLOBAL_SLIDING 4096 GQA 16:4 d=128, then CAUSAL 3000 MHA 64:64 d=64", flush=True)
    s1 = _case("GLOBAL_SLIDING", 4096, 16, 4, 128, seed=41)  # cut dK/dV columns: fp32 sums in the workspace
    s2 = _case("CAUSAL", 3000, 64, 64, 64, seed=42)          # one workgroup per column, over the stale sums
    print(f"kv splits: {s1}, {s2}", flush=True)
    assert s1 > 1 and s2 == 1


def test_static_workspace_refuses_oversized_call():
    """64 heads x 256K query rows need 128 MiB of row vectors: refused with a clear message, nothing
    launched (the pointers are never dereferenced)."""
    import mask_aware_dense_amd as mad
    T = 262144
    plan = mad.mask_compile(mad.mask_slices("CAUSAL", T), T, T).upload()
    assert mad.bwd_workspace_bytes(plan, T, T, 64, 8, 128) > mad.STATIC_WORKSPACE_BYTES
    p = ctypes.c_void_p(1 << 20)
    L = mad.lib()
    st = L.mad_attn_bwd_static(plan.handle, p, p, p, p, p, p, p, p, p, T, T, 64, 8, 128, None, ctypes.c_float(0.1),
                               None)
    assert st == 2 and b"static workspace" in L.mad_last_error()
