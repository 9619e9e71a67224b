"""Graph capture and the autograd wrapper.

The layer's entry points enqueue kernels only (no memset, copy or synchronisation), so a whole
step - pool, route, inversion, attention forward, and the backward - can be captured in one HIP
graph. Each replay must equal the eager result bit for bit, with eager work and synchronisation
between the replays and new inputs written into the captured buffers. The autograd wrapper must
give moc_attend_bwd's gradients."""
import pytest
import torch

import moc_inputs as mi
from test_gpu_parity import _say

pytestmark = pytest.mark.gpu


def test_layer_step_replays_equal_eager():
    import sparse_chunk_routed_amd as moc
    dev = torch.device("cuda:0")
    w = mi.grad_slice()
    Q, K, V, dO = (x.to(dev) for x in mi.make_qkv(w, with_dout=True))
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    cfg = moc.RouteCfg(w.top_k, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed)

    def step():
        kbar = moc.pool_keys(K, lay)
        sel, nsel = moc.route(Q, kbar, lay, cfg)
        vl = moc.build_varlen(sel, nsel, lay, cfg, w.d, Q.dtype)
        O, lse = moc.attend_fwd(Q, K, V, lay, vl)
        dQ, dK, dV = moc.attend_bwd(Q, K, V, O, lse, dO, lay, vl)
        return sel, O, lse, dQ, dK, dV

    step()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            outs = step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(3):
        # new inputs in the captured buffers (eager work between replays)
        gen = torch.Generator(device="cpu").manual_seed(100 + r)
        for x in (Q, K, V, dO):
            x.copy_((torch.randn(x.shape, generator=gen) * 0.5).to(x.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = step()
        torch.cuda.synchronize()
        for name, a, b in zip(("sel", "O", "lse", "dQ", "dK", "dV"), outs, ref):
            assert torch.equal(a, b), (r, name)
        _say(f"replay {r}: sel, O, lse, dQ, dK, dV equal the eager step")


def test_autograd_function_matches_entry_points_and_oracle():
    """MoCAttention (torch.autograd.Function): the forward is moc_attend_fwd over the routed
    sets, the gradients are moc_attend_bwd's (bit for bit) and match the oracle's backward."""
    import numpy as np
    import sparse_chunk_routed_amd as moc
    from oracle import moc_oracle as mo
    dev = torch.device("cuda:0")
    w = mi.grad_slice()
    Q, K, V, dO = mi.make_qkv(w, with_dout=True)
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    cfg = moc.RouteCfg(w.top_k, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed)
    Qd, Kd, Vd = (x.to(dev).requires_grad_(True) for x in (Q, K, V))
    O = moc.MoCAttention.apply(Qd, Kd, Vd, lay, cfg)
    O.backward(dO.to(dev))
    r = moc.forward(Qd.detach(), Kd.detach(), Vd.detach(), lay, cfg)
    gq, gk, gv = moc.attend_bwd(Qd.detach(), Kd.detach(), Vd.detach(), r.O, r.lse, dO.to(dev),
                                lay, r.varlen)
    torch.cuda.synchronize()
    assert torch.equal(O.detach(), r.O)
    for a, b in ((Qd.grad, gq), (Kd.grad, gk), (Vd.grad, gv)):
        assert torch.equal(a, b)
    sel = r.sel.cpu().numpy()
    rq, rk, rv = mo.attend_bwd(Q, K, V, dO, w.layout, sel)
    for name, a, b in (("dQ", Qd.grad, rq), ("dK", Kd.grad, rk), ("dV", Vd.grad, rv)):
        err = float(np.max(np.abs(a.float().cpu().numpy() - b)))
        _say(f"autograd {name}: max|err| vs oracle {err:.3e}")
        assert err <= 1e-2
