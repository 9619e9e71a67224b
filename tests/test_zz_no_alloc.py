"""moc_route_noalloc - the routing entry point for callers that cannot allocate (its kbar split
lives in a static device buffer) - against moc_route with a caller workspace, through the C
ABI: selections bit for bit, on calls in a row whose inputs shrink (the buffer keeps the last
call's contents)."""
import ctypes

import pytest
import torch

import moc_inputs as mi
from test_gpu_parity import _say

pytestmark = pytest.mark.gpu


def _compare(w):
    import sparse_chunk_routed_amd as moc
    L = moc._lib
    lib = L.load()
    dev = torch.device("cuda:0")
    Q, K = (x.to(dev) for x in mi.make_qkv(w)[:2])
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    cfg = moc.RouteCfg(w.top_k, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed)
    kbar = moc.pool_keys(K, lay)
    ref_sel, ref_nsel = moc.route(Q, kbar, lay, cfg)
    sel = torch.full_like(ref_sel, -5)
    nsel = torch.full_like(ref_nsel, -5)
    B, H, Lt, d = Q.shape
    s = lay.struct(B, H, d, Q.dtype)
    st = torch.cuda.current_stream(dev).cuda_stream
    L.check(lib.moc_route_noalloc(ctypes.byref(s), ctypes.byref(cfg.struct()),
                                  ctypes.c_void_p(Q.data_ptr()), ctypes.c_void_p(kbar.data_ptr()),
                                  ctypes.c_void_p(sel.data_ptr()) if sel.numel() else None,
                                  ctypes.c_void_p(nsel.data_ptr()), st))
    torch.cuda.synchronize()
    assert torch.equal(sel, ref_sel) and torch.equal(nsel, ref_nsel)
    scratch = B * H * w.C * d * 6 if Q.dtype == torch.bfloat16 else 0
    _say(f"{w.name}: L={Lt} H={H} C={w.C} {Q.dtype}: moc_route_noalloc equals moc_route "
         f"({int(nsel.sum())} selections, {scratch} bytes of static scratch)")


def test_route_noalloc_equals_route_on_shrinking_calls():
    _compare(mi.train())                 # 175,232 tokens, 12 heads, noise: 1.0 MB of scratch
    _compare(mi.grad_slice(H=2))         # smaller: the buffer still holds the first call's terms
    _compare(mi.tiny())                  # fp32 queries score without the split: no scratch
