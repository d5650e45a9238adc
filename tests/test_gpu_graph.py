"""The forward and backward captured in a HIP graph and replayed.

Every launch of the path is a kernel (the work-claim counters are cleared by a kernel, not a memset), so
the whole step can be captured.  The graph is replayed several times, with eager work (refilling the
outputs) and synchronisations between the replays, and every replay is compared with the eager result:
bit-exact for O, LSE, dQ, dK and dV (CAUSAL 4K GQA 64:32 keeps one workgroup per dK/dV column, so nothing
is summed in arrival order)."""
import numpy as np
import pytest

from mad_inputs import grad_out, qkv

pytestmark = pytest.mark.gpu


def test_fwd_bwd_graph_replays_match_eager():
    import torch
    import mask_aware_dense_amd as mad
    T, Hq, Hkv, d = 4096, 64, 32, 128
    plan = mad.mask_compile(mad.mask_slices("CAUSAL", T), T, T).upload()
    assert mad.bwd_kv_splits(plan, Hq, Hkv) == 1
    dev = torch.device("cuda", 0)
    q, k, v = (x.to(dev) for x in qkv(41, T, T, Hq, Hkv, d))
    do = grad_out(41, T, Hq, d).to(dev)
    scale = 1.0 / np.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fws = torch.empty(mad.FWD_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    ws = torch.empty(mad.bwd_workspace_bytes(plan, T, T, Hq, Hkv, d), dtype=torch.uint8, device=dev)
    outs = (o, lse, dq, dk, dv)

    def step():
        mad.attn_fwd(plan, q, k, v, o, lse, scale, workspace=fws)
        mad.attn_bwd(plan, q, k, v, o, do, lse, dq, dk, dv, ws, scale)

    def refill():
        for t in outs:
            t.fill_(float("nan"))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    refill()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        refill()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(("o", "lse", "dq", "dk", "dv"), outs, eager):
            assert torch.equal(t, e), f"replay {rep}: {name} differs from the eager result"
