"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle.  Inputs come from mad_inputs; expected values from
oracle/ only."""
import numpy as np

# Tolerances of the parity bar: O and LSE max-abs 2e-2 and relative L2 1e-2;
# dQ, dK, dV max-abs 5e-2 and relative L2 2e-2; -inf LSE rows must match exactly.
TOL_FWD = (2e-2, 1e-2)
TOL_BWD = (5e-2, 2e-2)


def torch_mod():
    import torch
    return torch


def spec_kwargs(spec):
    """mask_slices keyword arguments equivalent to an oracle MaskSpec (pattern parameters only)."""
    kw = dict(window=spec.window, question=spec.question, n_answers=spec.n_answers,
              global_len=spec.global_len, block=spec.block)
    if spec.prefix is not None:
        kw["prefix"] = spec.prefix
    if spec.doc_lens and spec.pattern != "SHARED_QUESTION":  # the C ABI reads doc_lens as answer lengths there
        kw["doc_lens"] = list(spec.doc_lens)
    if spec.answer_lens:
        kw["answer_lens"] = list(spec.answer_lens)
    return kw


def gpu_attention(plan, q, k, v, do, scale, bwd=True, o_in=None, lse_in=None, fill=float("nan")):
    """Run fwd (and bwd) on cuda:0.  q, k, v, do are CPU bf16 tensors.  Returns CPU float64 arrays.
    fill: the value the output buffers hold before the calls (NaN, so that an element the kernels
    leave unwritten fails the comparison; None leaves torch.empty's contents)."""
    import mask_aware_dense_amd as mad
    torch = torch_mod()
    dev = torch.device("cuda", 0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    Tq, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    plan.upload()
    def out_like(shape, dtype):
        t = torch.empty(shape, dtype=dtype, device=dev)
        return t if fill is None else t.fill_(fill)
    o = out_like((Tq, Hq, d), torch.bfloat16)
    lse = out_like((Hq, Tq), torch.float32)
    fws = torch.empty(mad.FWD_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)  # the forward claims its items
    mad.attn_fwd(plan, qd, kd, vd, o, lse, scale, workspace=fws)
    out = {}
    if bwd:
        dod = do.to(dev)
        oi = o if o_in is None else o_in.to(dev)
        li = lse if lse_in is None else lse_in.to(dev)
        dq = out_like(tuple(qd.shape), torch.bfloat16)
        dk = out_like(tuple(kd.shape), torch.bfloat16)
        dv = out_like(tuple(vd.shape), torch.bfloat16)
        ws = torch.empty(max(mad.bwd_workspace_bytes(plan, Tq, Tk, Hq, Hkv, d), 256), dtype=torch.uint8, device=dev)
        mad.attn_bwd(plan, qd, kd, vd, oi, dod, li, dq, dk, dv, ws, scale)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    out.update(o=o, lse=lse)
    return {n: t.detach().float().cpu().numpy().astype(np.float64) for n, t in out.items()}


def check_close(name, got, ref, tol, mask=None):
    """Assert max-abs and relative-L2 error within tol = (max_abs, rel_l2)."""
    a = np.asarray(got, dtype=np.float64)
    b = np.asarray(ref, dtype=np.float64)
    assert a.shape == b.shape, (name, a.shape, b.shape)
    if mask is not None:
        a, b = a[mask], b[mask]
    assert np.all(np.isfinite(a)), f"{name}: non-finite values"
    err = np.abs(a - b)
    mx = float(err.max()) if err.size else 0.0
    nb = float(np.linalg.norm(b))
    rel = float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))
    assert mx <= tol[0] and rel <= tol[1], f"{name}: max_abs {mx:.3e} (tol {tol[0]}), rel_l2 {rel:.3e} (tol {tol[1]})"
    return mx, rel


def check_lse(got, ref):
    ninf_g, ninf_r = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), "LSE -inf rows differ"
    fin = ~ninf_r
    return check_close("lse", got, ref, TOL_FWD, mask=fin)
