"""GPU parity of outer-loop context routing (Mixture of Contexts summary, Appendix I) through the
C ABI (moc_route_outer, moc_route_masked) against the oracle.

Bars: coarse segment selections identical as sets except where the oracle's M-th vs (M+1)-th
segment score gap is below 1e-4 relative; the candidate mask bit-exact given the selections;
inner selections (with and without drop noise) identical except tie-exempt queries, against the
oracle run on the mask of the GPU's coarse selections; pair counts exact.
"""
import numpy as np
import pytest
import torch

import moc_inputs as mi
import parity_checks as pc
from oracle import moc_oracle as mo
from test_gpu_parity import _say

pytestmark = pytest.mark.gpu


def _mask_from_seg_sel(seg_sel, seg_nsel, seg_chunk, C):
    """bool [B,H,C,C] from coarse selections: own segment plus picked segments."""
    so = np.asarray(seg_chunk)
    seg_of = np.repeat(np.arange(len(so) - 1), np.diff(so))
    B, H, nseg, _ = seg_sel.shape
    allowed = np.zeros((B, H, nseg, nseg), dtype=bool)
    for b in range(B):
        for h in range(H):
            for s in range(nseg):
                allowed[b, h, s, s] = True
                allowed[b, h, s, seg_sel[b, h, s, :seg_nsel[b, h, s]]] = True
    return allowed[:, :, seg_of][:, :, :, seg_of]


def _bits_to_bool(words, C):
    w = words.view(np.uint32)
    bits = (w[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(*w.shape[:-1], -1)[..., :C].astype(bool)


def _run(w, seg_chunk, M, causal, noise=False):
    import sparse_chunk_routed_amd as moc
    dev = torch.device("cuda:0")
    Q, K = mi.make_qkv(w)[:2]
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    Qd, Kd = Q.to(dev), K.to(dev)
    out = moc.route_outer(Qd, Kd, lay, seg_chunk, M, causal)
    cfg = moc.RouteCfg(w.top_k, causal, w.p_max if noise else 0.0, w.lam if noise else 0.0,
                       w.max_drop_in, w.seed)
    kbar = moc.pool_keys(Kd, lay)
    sel, nsel = moc.route(Qd, kbar, lay, cfg, cand_mask=out.cand_mask)
    vl = moc.build_varlen(sel, nsel, lay, cfg, w.d, Qd.dtype)
    torch.cuda.synchronize()
    return dict(Q=Q, K=K, seg_sel=out.seg_sel.cpu().numpy(), seg_nsel=out.seg_nsel.cpu().numpy(),
                cmask=out.cand_mask.cpu().numpy(), sel=sel.cpu().numpy(),
                nsel=nsel.cpu().numpy(), pairs=vl.pair_count.cpu().numpy(),
                kbar=kbar.cpu().numpy())


def _check(w, seg_chunk, M, causal, noise=False):
    g = _run(w, seg_chunk, M, causal, noise)
    lay = w.layout
    # coarse selections against the oracle (tie exemption)
    orr = mo.route_outer(g["Q"], g["K"], lay, seg_chunk, M, causal)
    same = np.all(np.sort(g["seg_sel"], -1) == np.sort(orr.seg_sel, -1), -1)
    same &= g["seg_nsel"] == orr.seg_nsel
    bad = ~same & ~orr.gap_exempt
    assert not bad.any(), np.argwhere(bad)[:5]
    _say(f"{w.name} M={M} causal={causal}: coarse selections equal "
         f"({int((~same).sum())} tie-exempt differ)")
    # the mask exactly encodes the GPU's coarse selections
    want = _mask_from_seg_sel(g["seg_sel"], g["seg_nsel"], seg_chunk, lay.C)
    assert np.array_equal(_bits_to_bool(g["cmask"], lay.C), want)
    # inner routing against the oracle restricted by that mask
    kb = mo.pool_keys(g["K"], lay)
    assert np.array_equal(g["kbar"].view(np.uint32), kb.view(np.uint32))
    r = mo.route(g["Q"], kb, lay, w.top_k, causal, cand_mask=want)
    if noise:
        osel, onsel = mo.drop_noise(r, lay, causal, w.p_max, w.lam, w.max_drop_in, w.seed,
                                    cand_mask=want)
    else:
        osel, onsel = r.sel, r.nsel
    gs = g["sel"][..., :osel.shape[-1]]
    same = np.all(gs == osel, -1) & (g["nsel"] == onsel)
    bad = ~same & ~r.gap_exempt
    assert not bad.any(), (np.argwhere(bad)[:5], gs[tuple(np.argwhere(bad)[0])],
                           osel[tuple(np.argwhere(bad)[0])])
    mo.check_routing(lay, g["sel"], g["nsel"], w.top_k, causal, exact_count=not noise,
                     cand_mask=want)
    assert np.array_equal(g["pairs"], mo.pair_counts(lay, g["sel"]))
    _say(f"{w.name}: inner selections equal ({int((~same).sum())} tie-exempt differ), "
         f"pairs {int(g['pairs'].sum())}")
    return g


@pytest.mark.parametrize("M,causal", [(1, True), (2, True), (2, False)])
def test_outer_tiny_fp32(M, causal):
    w = mi.tiny()
    _check(w, [0, 1, 5, 9, 13, 17], M, causal)


def test_outer_slice_bf16_with_noise():
    """bf16, 12 heads, the persistent router with drop-off / drop-in inside the mask."""
    w = mi.grad_slice()
    _check(w, [0, 1, 5, 9, 13, 17], 1, True, noise=True)
    _check(w, [0, 1, 3, 7, 10, 17], 2, False, noise=True)


def test_outer_many_chunks_bf16():
    """C = 201 (> 128): the per-tile router with the mask; segments of two shots."""
    sizes = [32] + [16] * 200
    shots = [-1] + [i // 20 for i in range(200)]
    lay = mi.layout_from_chunks(sizes, shots)
    w = mi.Workload("c201", 1, 2, 64, "bf16", lay, top_k=3, causal=True, clustered_keys=True,
                    seed=5)
    segs = [0, 1] + [1 + 40 * i for i in range(1, 6)]
    _check(w, segs, 2, True)


def test_outer_all_segments_equals_plain_routing():
    """M >= nseg admits every candidate: the masked router returns the plain router's result."""
    import sparse_chunk_routed_amd as moc
    w = mi.grad_slice()
    dev = torch.device("cuda:0")
    Q, K = mi.make_qkv(w)[:2]
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    Qd, Kd = Q.to(dev), K.to(dev)
    segs = [0, 1, 5, 9, 13, 17]
    out = moc.route_outer(Qd, Kd, lay, segs, len(segs), True)
    cfg = moc.RouteCfg(w.top_k, True, 0.3, 1.0, w.max_drop_in, w.seed)
    kbar = moc.pool_keys(Kd, lay)
    a = moc.route(Qd, kbar, lay, cfg)
    b = moc.route(Qd, kbar, lay, cfg, cand_mask=out.cand_mask)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_outer_headline_full_size():
    """The headline_outer workload the benchmark times (175,232 tokens, 12 heads, one segment per
    shot and the text, M = 2, inner top-2): coarse selections of every (head, query segment)
    against the oracle's, the candidate mask bit-exact, every inner selection against the
    oracle's masked routing (tie exemption, legality within the mask), pair counts exact, and the
    attention on sampled rows of every head."""
    import sparse_chunk_routed_amd as moc
    w = mi.headline_outer()
    dev = torch.device("cuda:0")
    Q, K, V = mi.make_qkv(w)
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    Qd, Kd, Vd = Q.to(dev), K.to(dev), V.to(dev)
    out = moc.route_outer(Qd, Kd, lay, w.segments, w.outer_M, w.causal)
    cfg = moc.RouteCfg(w.top_k, w.causal, 0.0, 0.0, w.max_drop_in, w.seed)
    kbar = moc.pool_keys(Kd, lay)
    sel, nsel = moc.route(Qd, kbar, lay, cfg, cand_mask=out.cand_mask)
    vl = moc.build_varlen(sel, nsel, lay, cfg, w.d, Qd.dtype)
    O, lse = moc.attend_fwd(Qd, Kd, Vd, lay, vl)
    torch.cuda.synchronize()
    g_seg, g_nseg = out.seg_sel.cpu().numpy(), out.seg_nsel.cpu().numpy()
    orr = mo.route_outer(Q, K, w.layout, w.segments, w.outer_M, w.causal)
    same = np.all(np.sort(g_seg, -1) == np.sort(orr.seg_sel, -1), -1) & (g_nseg == orr.seg_nsel)
    assert not (~same & ~orr.gap_exempt).any(), np.argwhere(~same)[:5]
    _say(f"coarse selections: {int(same.sum())}/{same.size} equal, "
         f"{int((~same).sum())} tie-exempt differ")
    want = _mask_from_seg_sel(g_seg, g_nseg, w.segments, w.C)
    assert np.array_equal(_bits_to_bool(out.cand_mask.cpu().numpy(), w.C), want)
    kb = mo.pool_keys(K, w.layout)
    assert np.array_equal(kbar.cpu().numpy().view(np.uint32), kb.view(np.uint32))
    r = mo.route(Q, kb, w.layout, w.top_k, w.causal, cand_mask=want)
    hsel, hnsel = sel.cpu().numpy(), nsel.cpu().numpy()
    pc.check_selection(w.layout, hsel, hnsel, r.sel, r.nsel, r, Q, kb, w.causal,
                       label="headline_outer inner")
    pc.check_legal(w.layout, hsel, hnsel, w.top_k, w.causal, cand_mask=want)
    assert np.array_equal(vl.pair_count.cpu().numpy(), mo.pair_counts(w.layout, hsel))
    rng = np.random.default_rng(11)
    rows = [(0, h, int(t)) for h in range(w.H) for t in rng.choice(w.L, 16, replace=False)]
    Oo, lo = mo.attend(Q, K, V, w.layout, hsel, rows=rows)
    hO, hl = O.float().cpu().numpy(), lse.cpu().numpy()
    err = float(np.max(np.abs(np.stack([hO[row] for row in rows]) - Oo)))
    lerr = float(np.max(np.abs(np.array([hl[row] for row in rows]) - lo)))
    _say(f"headline_outer attention rows={len(rows)} max|dO|={err:.3e} max|dlse|={lerr:.3e}")
    assert err <= 1e-2 and lerr <= 1e-2
