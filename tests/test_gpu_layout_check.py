"""GPU tests of the device layout check (moc_layout.check), through the C ABI.

* Valid layouts with the check on: every entry point gives bit-identical outputs to the same
  calls without the check, and the word stays 0.
* A word that is already non-zero (set by the test on a valid layout): every entry point
  leaves its outputs untouched and keeps the word - each kernel returns at its start.
* The check kernel alone (moc_check_layout, which launches nothing else and reads only the C+1
  offsets and C shot ids) on malformed layouts reports the same bits as the host build of the
  check. No other kernel ever sees a malformed layout.
"""
import ctypes

import numpy as np
import pytest
import torch

import moc_inputs as mi
from test_gpu_parity import _say

pytestmark = pytest.mark.gpu


def _moc():
    import sparse_chunk_routed_amd as moc
    return moc


def _layout(w, check: bool):
    moc = _moc()
    return moc.DeviceLayout.from_layout(w.layout, torch.device("cuda:0")) if not check else \
        moc.DeviceLayout(w.layout.chunk_offsets, w.layout.chunk_shot, w.layout.text_begin,
                         w.layout.text_end, device=torch.device("cuda:0"), device_check=True)


def _layer(w, lay, Q, K, V, dO):
    """pool -> route -> varlen -> forward -> backward, outer routing and MXFP8 quantisation."""
    moc = _moc()
    cfg = moc.RouteCfg(w.top_k, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed)
    r = moc.forward(Q, K, V, lay, cfg)
    dQ, dK, dV = moc.attend_bwd(Q, K, V, r.O, r.lse, dO, lay, r.varlen)
    outer = moc.route_outer(Q, K, lay, [0, 1, 5, 9, 13, 17], 2, True)
    qm = moc.mx_quantize(Q, lay)
    torch.cuda.synchronize()
    return [r.kbar, r.sel, r.nsel, r.O, r.lse, r.varlen.pair_count, dQ, dK, dV, outer.seg_sel,
            outer.cand_mask, qm.codes, qm.scales]


def test_check_on_valid_layout_changes_nothing():
    w = mi.grad_slice(H=2)
    Q, K, V, dO = (x.cuda() for x in mi.make_qkv(w, with_dout=True))
    ref = _layer(w, _layout(w, False), Q, K, V, dO)
    lay = _layout(w, True)
    got = _layer(w, lay, Q, K, V, dO)
    assert int(lay.check_word.item()) == 0
    lay.check_status()  # no error
    for i, (a, b) in enumerate(zip(ref, got)):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.bool else a,
                           b.view(torch.uint8) if b.dtype != torch.bool else b), i
    _say(f"checked layer equals unchecked layer ({len(ref)} outputs, bit for bit)")


def test_nonzero_word_skips_every_kernel():
    """The word is set by the test (bit MOC_LAYOUT_BAD_END) on a valid layout; no call may
    write its outputs."""
    moc = _moc()
    L = moc._lib
    lib = L.load()
    w = mi.grad_slice(H=2)
    Q, K, V, dO = (x.cuda() for x in mi.make_qkv(w, with_dout=True))
    good = _layout(w, False)
    cfg = moc.RouteCfg(w.top_k, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed)
    r = moc.forward(Q, K, V, good, cfg)  # a valid varlen for the attention calls below
    torch.cuda.synchronize()
    lay = _layout(w, True)
    lay.check_word.fill_(L.MOC_LAYOUT_BAD_END)
    B, H, Lt, d = Q.shape
    s = lay.struct(B, H, d, Q.dtype)
    st = torch.cuda.current_stream().cuda_stream
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    kbar = torch.full((B, H, w.C, d), 7.0, device="cuda")
    L.check(lib.moc_pool_keys(ctypes.byref(s), p(K), p(kbar), st))
    S = moc.sel_width(cfg, w.C)
    sel = torch.full((B, H, Lt, S), -7, dtype=torch.int32, device="cuda")
    nsel = torch.full((B, H, Lt), -7, dtype=torch.int32, device="cuda")
    rws = torch.empty(moc.workspace_bytes(lay, B, H, d, Q.dtype, cfg, L.MOC_OP_ROUTE),
                      dtype=torch.uint8, device="cuda")
    L.check(lib.moc_route(ctypes.byref(s), ctypes.byref(cfg.struct()), p(Q), p(r.kbar), p(sel),
                          p(nsel), p(rws), rws.numel(), st))
    vws = torch.empty(moc.workspace_bytes(lay, B, H, d, Q.dtype, cfg, L.MOC_OP_VARLEN),
                      dtype=torch.uint8, device="cuda")
    pairs = torch.full((B, H), -7, dtype=torch.int64, device="cuda")
    vs = L.MocVarlen()
    L.check(lib.moc_build_varlen(ctypes.byref(s), ctypes.byref(cfg.struct()), p(r.sel),
                                 p(r.nsel), ctypes.byref(vs), p(pairs), p(vws), vws.numel(), st))
    O = torch.full_like(Q, 7.0)
    lse = torch.full((B, H, Lt), 7.0, device="cuda")
    fws = torch.empty(moc.workspace_bytes(lay, B, H, d, Q.dtype, cfg, L.MOC_OP_FWD),
                      dtype=torch.uint8, device="cuda")
    L.check(lib.moc_attend_fwd(ctypes.byref(s), ctypes.byref(r.varlen.struct), p(Q), p(K), p(V),
                               ctypes.c_float(d ** -0.5), p(O), p(lse), p(fws), fws.numel(), st))
    grads = [torch.full_like(Q, 7.0) for _ in range(3)]
    bws = torch.empty(moc.workspace_bytes(lay, B, H, d, Q.dtype, cfg, L.MOC_OP_BWD),
                      dtype=torch.uint8, device="cuda")
    L.check(lib.moc_attend_bwd(ctypes.byref(s), ctypes.byref(r.varlen.struct), p(Q), p(K), p(V),
                               p(r.O), p(r.lse), p(dO), ctypes.c_float(d ** -0.5),
                               *(p(x) for x in grads), p(bws), bws.numel(), st))
    Lp = (Lt + 63) // 64 * 64
    codes = torch.full((B, H, Lp, d), 7, dtype=torch.uint8, device="cuda")
    scales = torch.full((B, H, Lp, d // 32), 7, dtype=torch.uint8, device="cuda")
    L.check(lib.moc_mx_quantize(ctypes.byref(s), p(Q), p(codes), p(scales), st))
    segs = torch.tensor([0, 1, 5, 9, 13, 17], dtype=torch.int32, device="cuda")
    seg_sel = torch.full((B, H, 5, 2), -7, dtype=torch.int32, device="cuda")
    seg_nsel = torch.full((B, H, 5), -7, dtype=torch.int32, device="cuda")
    cmask = torch.full((B, H, w.C, 1), -7, dtype=torch.int32, device="cuda")
    ows = torch.empty(moc.workspace_bytes(lay, B, H, d, Q.dtype, cfg, L.MOC_OP_OUTER),
                      dtype=torch.uint8, device="cuda")
    L.check(lib.moc_route_outer(ctypes.byref(s), p(segs), 5, 2, 1, p(Q), p(K), p(seg_sel),
                                p(seg_nsel), p(cmask), p(ows), ows.numel(), st))
    torch.cuda.synchronize()
    assert bool((kbar == 7.0).all())
    assert bool((sel == -7).all()) and bool((nsel == -7).all())
    assert bool((pairs == -7).all())
    assert bool((O == 7.0).all()) and bool((lse == 7.0).all())
    assert all(bool((x == 7.0).all()) for x in grads)
    assert bool((codes == 7).all()) and bool((scales == 7).all())
    assert bool((seg_sel == -7).all()) and bool((seg_nsel == -7).all())
    assert bool((cmask == -7).all())
    assert int(lay.check_word.item()) == L.MOC_LAYOUT_BAD_END
    with pytest.raises(moc.MocError) as e:
        lay.check_status()
    assert e.value.status == L.MOC_ELAYOUT
    # no routed-row total is reported for a rejected layout
    total = ctypes.c_int64(-7)
    assert lib.moc_varlen_total(ctypes.byref(s), ctypes.byref(r.varlen.struct), ctypes.byref(total),
                                st) == L.MOC_ELAYOUT
    assert total.value == -7
    _say("a non-zero check word kept every kernel from writing (8 entry points)")


def test_check_kernel_alone_matches_host_bits():
    """Malformed layouts given only to the check kernel (moc_check_layout): its word equals the
    host build's bits."""
    moc = _moc()
    L = moc._lib
    cases = []
    off = [0, 4, 10, 13, 20, 26]
    shot = [-1, 0, 0, 1, 1]
    cases.append(("valid", off, shot, 0, 4, 26))
    cases.append(("start", [1, 4, 10, 13, 20, 26], shot, 0, 4, 26))
    cases.append(("order", [0, 4, 10, 10, 20, 26], shot, 0, 4, 26))
    cases.append(("end", off, shot, 0, 4, 30))
    cases.append(("shot_id", off, [-1, 0, 0, -2, 1], 0, 4, 26))
    cases.append(("text_tag", off, [5, 0, 0, 1, 1], 0, 4, 26))
    cases.append(("straddle", off, shot, 0, 6, 26))
    cases.append(("shot_split", off, [-1, 0, 1, 0, 2], 0, 4, 26))
    rng = np.random.default_rng(9)
    for i in range(20):  # larger random layouts with a random shot id changed
        lay = mi.make_random_layout(rng, max_shots=30, max_frames=20, max_chunk=40)
        sh = np.array(lay.chunk_shot)
        j = int(rng.integers(0, len(sh)))
        sh[j] = int(rng.integers(-1, 30))
        cases.append((f"rand{i}", list(lay.chunk_offsets), list(sh), lay.text_begin,
                      lay.text_end, lay.L))
    n_flag = 0
    for name, o, sh, tb, te, Lt in cases:
        o32 = np.array(o, dtype=np.int32)
        s32 = np.array(sh, dtype=np.int32)
        want = int(L.load().moc_layout_check_host(o32.ctypes.data, s32.ctypes.data, len(s32), Lt,
                                                   tb, te))
        dl = moc.DeviceLayout(o32, s32, tb, te, device=torch.device("cuda:0"),
                              device_check=True, validate=False)
        dl.L = Lt
        dl.check_on_device()
        torch.cuda.synchronize()
        got = int(dl.check_word.item()) & 0xFFFFFFFF
        assert got == want, (name, got, want)
        n_flag += want != 0
    assert n_flag >= 7
    _say(f"check kernel alone: {len(cases)} layouts, {n_flag} flagged, bits equal to the host's")
