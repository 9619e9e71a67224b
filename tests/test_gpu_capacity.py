"""GPU tests of the attention workspaces sized from the real routing (moc_varlen_set_capacity,
moc_attend_workspace_bytes), through the C ABI.

* With the capacity set to the routing's total, forward and backward equal the default-capacity
  calls bit for bit, in smaller workspaces.
* With a capacity one row short, the guard of each attention call stops every kernel: outputs
  keep their prefilled values and moc_varlen_status reports MOC_EWORKSPACE.
* The train workload's FWD + BWD workspaces at its real capacity (printed).
"""
import pytest
import torch

import moc_inputs as mi
from test_gpu_parity import _say

pytestmark = pytest.mark.gpu


def _setup(w):
    import sparse_chunk_routed_amd as moc
    dev = torch.device("cuda:0")
    Q, K, V, dO = (x.to(dev) for x in mi.make_qkv(w, with_dout=True))
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    cfg = moc.RouteCfg(w.top_k, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed)
    kbar = moc.pool_keys(K, lay)
    sel, nsel = moc.route(Q, kbar, lay, cfg)
    vl = moc.build_varlen(sel, nsel, lay, cfg, w.d, Q.dtype)
    return moc, lay, vl, Q, K, V, dO


def test_exact_capacity_equals_default():
    w = mi.grad_slice()
    moc, lay, vl, Q, K, V, dO = _setup(w)
    L = moc._lib
    O0, lse0 = moc.attend_fwd(Q, K, V, lay, vl)
    g0 = moc.attend_bwd(Q, K, V, O0, lse0, dO, lay, vl)
    big = (vl.workspace_bytes(L.MOC_OP_FWD), vl.workspace_bytes(L.MOC_OP_BWD))
    total = vl.total()
    assert total == int(vl.bucket_off()[-1].item())
    vl.set_capacity(total)
    small = (vl.workspace_bytes(L.MOC_OP_FWD), vl.workspace_bytes(L.MOC_OP_BWD))
    assert small[0] < big[0] and small[1] < big[1]
    O1, lse1 = moc.attend_fwd(Q, K, V, lay, vl)
    g1 = moc.attend_bwd(Q, K, V, O1, lse1, dO, lay, vl)
    vl.check_status()
    assert torch.equal(O0, O1) and torch.equal(lse0, lse1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)
    _say(f"slice: {total} routed rows of {vl.struct.routed_max}; FWD+BWD workspace "
         f"{sum(big) / 2**20:.1f} MiB -> {sum(small) / 2**20:.1f} MiB, outputs bit-identical")


def test_capacity_one_short_writes_nothing():
    import ctypes
    w = mi.grad_slice(H=2)
    moc, lay, vl, Q, K, V, dO = _setup(w)
    L = moc._lib
    lib = L.load()
    total = vl.total()
    assert total > 0
    vl.set_capacity(total - 1)
    B, H, Lt, d = Q.shape
    s = lay.struct(B, H, d, Q.dtype)
    st = torch.cuda.current_stream().cuda_stream
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    O = torch.full_like(Q, 7.0)
    lse = torch.full((B, H, Lt), 7.0, device=Q.device)
    fws = torch.empty(vl.workspace_bytes(L.MOC_OP_FWD), dtype=torch.uint8, device=Q.device)
    L.check(lib.moc_attend_fwd(ctypes.byref(s), ctypes.byref(vl.struct), p(Q), p(K), p(V),
                               ctypes.c_float(d ** -0.5), p(O), p(lse), p(fws), fws.numel(), st))
    with pytest.raises(moc.MocError) as e:
        vl.check_status()
    assert e.value.status == L.MOC_EWORKSPACE
    assert bool((O == 7.0).all()) and bool((lse == 7.0).all())
    grads = [torch.full_like(Q, 7.0) for _ in range(3)]
    bws = torch.empty(vl.workspace_bytes(L.MOC_OP_BWD), dtype=torch.uint8, device=Q.device)
    L.check(lib.moc_attend_bwd(ctypes.byref(s), ctypes.byref(vl.struct), p(Q), p(K), p(V), p(Q),
                               p(lse), p(dO), ctypes.c_float(d ** -0.5), *(p(x) for x in grads),
                               p(bws), bws.numel(), st))
    with pytest.raises(moc.MocError) as e:
        vl.check_status()
    assert e.value.status == L.MOC_EWORKSPACE
    assert all(bool((x == 7.0).all()) for x in grads)
    # a workspace below the capacity's size is refused on the host
    assert lib.moc_attend_fwd(ctypes.byref(s), ctypes.byref(vl.struct), p(Q), p(K), p(V),
                              ctypes.c_float(d ** -0.5), p(O), p(lse), p(fws), fws.numel() - 256,
                              st) == L.MOC_EWORKSPACE
    # back at the routing's total the calls run again
    vl.set_capacity(total)
    O2, _ = moc.attend_fwd(Q, K, V, lay, vl)
    vl.check_status()
    assert not bool((O2 == 7.0).all())
    _say(f"capacity {total - 1} < {total} routed rows: forward and backward wrote nothing")


def test_train_workspace_at_real_capacity():
    w = mi.train()
    moc, lay, vl, Q, K, V, dO = _setup(w)
    L = moc._lib
    route_b = moc.workspace_bytes(lay, w.B, w.H, w.d, Q.dtype, vl.cfg, L.MOC_OP_ROUTE)
    var_b = vl.ws.numel()
    big = (vl.workspace_bytes(L.MOC_OP_FWD), vl.workspace_bytes(L.MOC_OP_BWD))
    total = vl.total()
    vl.set_capacity(total)
    small = (vl.workspace_bytes(L.MOC_OP_FWD), vl.workspace_bytes(L.MOC_OP_BWD))
    _say(f"train: {total} routed rows of {vl.struct.routed_max} (S = {vl.S}); FWD "
         f"{big[0] / 1e9:.2f} -> {small[0] / 1e9:.2f} GB, BWD {big[1] / 1e9:.2f} -> "
         f"{small[1] / 1e9:.2f} GB; ROUTE {route_b / 1e6:.1f} MB, VARLEN {var_b / 1e6:.1f} MB")
    assert sum(small) < 0.5 * sum(big)
    O, lse = moc.attend_fwd(Q, K, V, lay, vl)
    moc.attend_bwd(Q, K, V, O, lse, dO, lay, vl)
    vl.check_status()
