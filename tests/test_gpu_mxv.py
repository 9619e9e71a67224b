"""GPU parity of the quantised-values variant (MXFP8 Q, K and V; moc_mx_quantize_v and
moc_attend_fwd_mxv) through the C ABI against the oracle.

Bars: the V tiles bit-exact against the oracle's key-axis quantisation (byte work; the tile
order and padding checked too). The attention against the oracle's exact attention over the
dequantised Q', K', V' (attend_mxv), per element within the oracle's bound on rounding the
softmax weights to e4m3 (pv_fp8_bound) plus 2^-8 |O| (bf16 output rounding) plus 1e-4 (fp32
arithmetic); lse, which the kernel takes from the unrounded weights, within the bf16 bar 1e-2
like the quantised-scores variant. With Q = 0 every weight is exactly 1, so the output is the
plain mean of V' over Omega(t) and the bound is 2^-8 |O| + 1e-4 alone. Bitwise deterministic.
"""
import numpy as np
import pytest
import torch

import moc_inputs as mi
from oracle import moc_oracle as mo
from test_gpu_parity import _sample_rows, _say

pytestmark = pytest.mark.gpu

ROW = 80


def _swap34(p):
    return (p & ~24) | ((p & 8) << 1) | ((p & 16) >> 1)


def _decode_tiles(vq: np.ndarray):
    """[B,H,T,d,80] tiles -> codes [B,H,d,64T] in key order and scales [B,H,d,2T]."""
    B, H, T, d, _ = vq.shape
    t = np.transpose(vq, (0, 1, 3, 2, 4))                       # [B,H,d,T,80]
    key_of_pos = np.array([32 * (q // 32) + _swap34(q % 32) for q in range(64)])
    codes = np.zeros((B, H, d, T, 64), np.uint8)
    codes[..., key_of_pos] = t[..., :64]
    return codes.reshape(B, H, d, 64 * T), t[..., 64:66].reshape(B, H, d, 2 * T), t[..., 66:]


def _special_columns(V: torch.Tensor) -> torch.Tensor:
    """Key blocks of head (0, 0) overwritten with cases the quantiser must get right: E4M3
    rounding ties (block max 256 fixes E = 0), values that round to +-0, an all-zero block,
    bf16 subnormals, magnitudes near the top of the range, a block spanning 1e-30 to 1e30."""
    V = V.clone()
    ties = [256.0, 17.0, 19.0, 2.0 ** -10, -(2.0 ** -10), -(2.0 ** -12), 1.5 * 2.0 ** -9,
            2.5 * 2.0 ** -9, -300.0, 448.0, 3.0, -0.0]
    col = torch.zeros(32)
    col[:len(ties)] = torch.tensor(ties)
    V[0, 0, :32, 0] = col.to(V.dtype)
    V[0, 0, :32, 1] = 0.0
    V[0, 0, 32:64, 2] = (torch.linspace(-1, 1, 32) * 1e-39).to(V.dtype)
    V[0, 0, :32, 3] = (torch.linspace(-1, 1, 32) * 3e38).to(V.dtype)
    V[0, 0, :16, 4] = 1e-30
    V[0, 0, 16:32, 4] = 1e30
    return V


@pytest.mark.parametrize("d", [64, 128])
def test_quantize_v_bit_exact(d):
    import sparse_chunk_routed_amd as moc
    dev = torch.device("cuda:0")
    lay = mi.make_random_layout(np.random.default_rng(11), max_shots=3, max_frames=3,
                                max_chunk=200)
    w = mi.Workload(f"mxv_q{d}", 2, 3, d, "bf16", lay, top_k=2, causal=True,
                    clustered_keys=False, seed=4)
    V = _special_columns(mi.make_qkv(w)[2])
    vq = moc.mx_quantize_v(V.to(dev), moc.DeviceLayout.from_layout(lay, dev))
    torch.cuda.synchronize()
    codes, scales, pad = _decode_tiles(vq.cpu().numpy())
    oc, osc = mo.mx_quantize_keys(V.float().numpy())
    L32 = oc.shape[-1]
    assert np.array_equal(codes[..., :L32], oc), np.argwhere(codes[..., :L32] != oc)[:5]
    assert np.array_equal(scales[..., :L32 // 32], osc)
    assert not codes[..., L32:].any() and not scales[..., L32 // 32:].any() and not pad.any()
    _say(f"{w.name}: L={w.L} (Lp={codes.shape[-1]}) V tiles bit-exact ({oc.size} codes)")


def _dequantised(Q, K, V, heads):
    """Q', K', V' of the listed (b, h) heads (zero elsewhere), as the kernel uses them."""
    Qd, Kd, Vd = (np.zeros(x.shape) for x in (Q, K, V))
    for b, h in heads:
        Qd[b, h] = mo.mx_dequantize(*mo.mx_quantize(Q[b, h].float().numpy()))
        Kd[b, h] = mo.mx_dequantize(*mo.mx_quantize(K[b, h].float().numpy()))
        Vd[b, h] = mo.mx_dequantize_keys(*mo.mx_quantize_keys(V[b, h].float().numpy()),
                                         V.shape[2])
    return Qd, Kd, Vd


def _mxv_run(w: mi.Workload, zero_q: bool = False):
    import sparse_chunk_routed_amd as moc
    dev = torch.device("cuda:0")
    Q, K, V = mi.make_qkv(w)
    if zero_q:
        Q = torch.zeros_like(Q)
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    cfg = moc.RouteCfg(w.top_k, w.causal, 0.0, 0.0, w.max_drop_in, w.seed)
    Qd, Kd, Vd = (x.to(dev) for x in (Q, K, V))
    kbar = moc.pool_keys(Kd, lay)
    sel, nsel = moc.route(Qd, kbar, lay, cfg)
    vl = moc.build_varlen(sel, nsel, lay, cfg, w.d, Qd.dtype)
    Qm, Km = moc.mx_quantize(Qd, lay), moc.mx_quantize(Kd, lay)
    Vq = moc.mx_quantize_v(Vd, lay)
    O, lse = moc.attend_fwd_mxv(Qm, Km, Vq, lay, vl)
    torch.cuda.synchronize()
    return dict(Q=Q, K=K, V=V, sel=sel.cpu().numpy(), O=O.float().cpu().numpy(),
                lse=lse.cpu().numpy())


def _compare(w, g, rows, zero_q=False):
    heads = sorted({(b, h) for b, h, _ in rows})
    Qd, Kd, Vd = _dequantised(g["Q"], g["K"], g["V"], heads)
    O, lse = mo.attend(Qd, Kd, Vd, w.layout, g["sel"], rows=rows)
    bound = 0.0 if zero_q else mo.pv_fp8_bound(Qd, Kd, Vd, w.layout, g["sel"], rows)
    tol = bound + 2.0 ** -8 * np.abs(O) + 1e-4
    got = np.stack([g["O"][b, h, t] for b, h, t in rows])
    gl = np.array([g["lse"][b, h, t] for b, h, t in rows])
    err = np.abs(got - O)
    lerr = float(np.max(np.abs(gl - lse)))
    _say(f"{w.name} quantised values: rows={len(rows)} max|dO|={err.max():.3e} mean "
         f"{err.mean():.3e}; largest share of the bound {np.max(err / tol):.3f}; "
         f"mean bound {np.mean(tol):.3e}; max|dlse|={lerr:.3e}")
    assert np.all(err <= tol), np.argwhere(err > tol)[:5]
    assert lerr <= 1e-2


def _all_rows(w):
    return [(b, h, t) for b in range(w.B) for h in range(w.H) for t in range(w.L)]


def test_zero_queries_average_the_values():
    """Q = 0: every weight is exactly 1 (exact in e4m3), O is the mean of V' over Omega(t)."""
    w = mi.grad_slice()
    g = _mxv_run(w, zero_q=True)
    _compare(w, g, [r for r in _all_rows(w) if r[1] in (0, 7)], zero_q=True)


def test_attend_mxv_slice():
    """The 4,224-token slice (12 heads, d = 128), every row of four heads."""
    w = mi.grad_slice()
    g = _mxv_run(w)
    _compare(w, g, [r for r in _all_rows(w) if r[1] in (0, 3, 6, 11)])


@pytest.mark.parametrize("seed", range(5))
def test_attend_mxv_random_layouts(seed):
    """Irregular chunks, B = 2, both head sizes, causal on and off, k from 0 to all,
    frame-is-shot, ragged L (L % 64 != 0); every row."""
    rng = np.random.default_rng(3000 + seed)
    lay = mi.make_random_layout(rng, max_shots=5, max_frames=4, max_chunk=300,
                                frame_is_shot=(seed == 3))
    d = 64 if seed in (0, 2) else 128
    w = mi.Workload(f"mxvrand{seed}", 2, 2, d, "bf16", lay,
                    top_k=min(lay.C, [1, 3, 0, lay.C, 2][seed]),
                    causal=seed in (0, 3, 4), clustered_keys=bool(seed != 2), seed=seed)
    _say(f"{w.name}: L={w.L} (L % 64 = {w.L % 64}) C={w.C} d={d}")
    _compare(w, _mxv_run(w), _all_rows(w))


def test_attend_mxv_headline_sampled():
    """The full-size headline workload; sampled rows (random and chunk edges) of three heads.
    Also reports how far quantising Q, K and V moves the output from the unquantised attention
    (a change of the function, bounded loosely here, not parity)."""
    w = mi.WORKLOADS["headline"]()
    g = _mxv_run(w)
    rows = [r for r in _sample_rows(w, 24) if r[1] in (0, 5, 11)]
    _compare(w, g, rows)
    O, lse = mo.attend(g["Q"], g["K"], g["V"], w.layout, g["sel"], rows=rows)
    got = np.stack([g["O"][b, h, t] for b, h, t in rows])
    d_o = np.abs(got - O)
    _say(f"quantisation effect vs unquantised attention: O max {d_o.max():.3e} mean "
         f"{d_o.mean():.3e} (|O| mean {np.abs(O).mean():.3e})")
    assert d_o.max() < 0.25


def test_attend_mxv_deterministic():
    w = mi.grad_slice()
    a, b = _mxv_run(w), _mxv_run(w)
    assert np.array_equal(a["O"].view(np.uint32), b["O"].view(np.uint32))
    assert np.array_equal(a["lse"].view(np.uint32), b["lse"].view(np.uint32))
