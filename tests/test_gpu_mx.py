"""GPU parity of the quantised-scores variant (MXFP8 Q and K, moc_mx_quantize and
moc_attend_fwd_mx) through the C ABI against the oracle.

Bars: codes and scales bit-exact (byte work), padded rows zero; the attention within the bf16
bar (max-abs 1e-2 on O and on lse) of the oracle's attention over the dequantised Q and K, on
the GPU's own routing (the routing itself is checked by the other parity tests); bitwise
deterministic.
"""
import numpy as np
import pytest
import torch

import moc_inputs as mi
from oracle import moc_oracle as mo
from test_gpu_parity import _sample_rows, _say

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _special_values(X: torch.Tensor) -> torch.Tensor:
    """Rows of X (bf16) overwritten with cases the quantiser must get right: an all-zero row,
    exact ties of the E4M3 rounding (block max 256 fixes E = 0), values that round to +-0,
    bf16 subnormals, and large magnitudes."""
    X = X.clone()
    d = X.shape[-1]
    X[0, 0, 1] = 0.0
    ties = [256.0, 17.0, 19.0, 2.0 ** -10, -(2.0 ** -10), -(2.0 ** -12), 1.5 * 2.0 ** -9,
            2.5 * 2.0 ** -9, -300.0, 449.0 - 1.0, 3.0, -0.0]
    row = torch.zeros(d)
    row[:len(ties)] = torch.tensor(ties)
    X[0, 0, 2] = row.to(X.dtype)
    X[0, 0, 3] = (torch.linspace(-1, 1, d) * 1e-39).to(X.dtype)      # bf16 subnormals
    X[0, 0, 4] = (torch.linspace(-1, 1, d) * 3e38).to(X.dtype)       # near the top of the range
    X[0, 0, 5, : d // 2] = 1e-30
    X[0, 0, 5, d // 2:] = 1e30
    return X


def _quant_check(X: torch.Tensor, w: mi.Workload):
    import sparse_chunk_routed_amd as moc
    dev = torch.device("cuda:0")
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    m = moc.mx_quantize(X.to(dev), lay)
    torch.cuda.synchronize()
    codes, scales = m.codes.cpu().numpy(), m.scales.cpu().numpy()
    oc, osc = mo.mx_quantize(X.float().numpy())
    L = X.shape[2]
    assert np.array_equal(codes[:, :, :L], oc), np.argwhere(codes[:, :, :L] != oc)[:5]
    assert np.array_equal(scales[:, :, :L], osc)
    assert not codes[:, :, L:].any() and not scales[:, :, L:].any()
    _say(f"{w.name}: MXFP8 codes and scales bit-exact ({oc.size} codes, L={L}, "
         f"Lp={codes.shape[2]})")


@pytest.mark.parametrize("d", [64, 128])
def test_quantize_bit_exact(d):
    lay = mi.make_random_layout(np.random.default_rng(7), max_shots=3, max_frames=3,
                                max_chunk=200)
    w = mi.Workload(f"mxq{d}", 2, 3, d, "bf16", lay, top_k=2, causal=True, clustered_keys=False,
                    seed=3)
    Q = mi.make_qkv(w)[0]
    _quant_check(_special_values(Q), w)


def _mx_run(w: mi.Workload):
    import sparse_chunk_routed_amd as moc
    dev = torch.device("cuda:0")
    Q, K, V = mi.make_qkv(w)
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    cfg = moc.RouteCfg(w.top_k, w.causal, 0.0, 0.0, w.max_drop_in, w.seed)
    Qd, Kd, Vd = (x.to(dev) for x in (Q, K, V))
    kbar = moc.pool_keys(Kd, lay)
    sel, nsel = moc.route(Qd, kbar, lay, cfg)
    vl = moc.build_varlen(sel, nsel, lay, cfg, w.d, Qd.dtype)
    Qm, Km = moc.mx_quantize(Qd, lay), moc.mx_quantize(Kd, lay)
    O, lse = moc.attend_fwd_mx(Qm, Km, Vd, lay, vl)
    torch.cuda.synchronize()
    return dict(Q=Q, K=K, V=V, sel=sel.cpu().numpy(), O=O.float().cpu().numpy(),
                lse=lse.cpu().numpy())


def _compare(w, g, rows=None):
    if rows is None:
        O, lse = mo.attend_mx(g["Q"], g["K"], g["V"], w.layout, g["sel"])
        err, lerr = np.max(np.abs(g["O"] - O)), np.max(np.abs(g["lse"] - lse))
    else:
        O, lse = mo.attend_mx(g["Q"], g["K"], g["V"], w.layout, g["sel"], rows=rows)
        got = np.stack([g["O"][b, h, t] for b, h, t in rows])
        gl = np.array([g["lse"][b, h, t] for b, h, t in rows])
        err, lerr = np.max(np.abs(got - O)), np.max(np.abs(gl - lse))
    _say(f"{w.name} quantised scores: max|dO|={err:.3e} max|dlse|={lerr:.3e}")
    assert err <= TOL and lerr <= TOL


def test_attend_mx_slice():
    """The 4,224-token slice (12 heads, d = 128), every row."""
    w = mi.grad_slice()
    _compare(w, _mx_run(w))


@pytest.mark.parametrize("seed", range(5))
def test_attend_mx_random_layouts(seed):
    """Irregular chunks, B = 2, both head sizes, causal on and off, k from 0 to all, frame-is-
    shot, ragged L (L % 64 != 0)."""
    rng = np.random.default_rng(2000 + seed)
    lay = mi.make_random_layout(rng, max_shots=5, max_frames=4, max_chunk=300,
                                frame_is_shot=(seed == 3))
    d = 64 if seed in (0, 2) else 128
    w = mi.Workload(f"mxrand{seed}", 2, 2, d, "bf16", lay,
                    top_k=min(lay.C, [1, 3, 0, lay.C, 2][seed]),
                    causal=seed in (0, 3, 4), clustered_keys=bool(seed != 2), seed=seed)
    _say(f"{w.name}: L={w.L} (L % 64 = {w.L % 64}) C={w.C} d={d}")
    _compare(w, _mx_run(w))


def test_attend_mx_headline_sampled():
    """The full-size headline workload in the launch configuration the benchmark times;
    sampled rows of three heads. Also reports how far quantising Q and K moves the output from
    the unquantised attention (a change of the function, bounded loosely here, not parity)."""
    w = mi.WORKLOADS["headline"]()
    g = _mx_run(w)
    rows = [r for r in _sample_rows(w, 24) if r[1] in (0, 5, 11)]
    _compare(w, g, rows)
    O, lse = mo.attend(g["Q"], g["K"], g["V"], w.layout, g["sel"], rows=rows)
    got = np.stack([g["O"][b, h, t] for b, h, t in rows])
    gl = np.array([g["lse"][b, h, t] for b, h, t in rows])
    d_o, d_l = np.abs(got - O), np.abs(gl - lse)
    _say(f"quantisation effect vs unquantised attention: O max {d_o.max():.3e} mean "
         f"{d_o.mean():.3e} (|O| mean {np.abs(O).mean():.3e}); lse max {d_l.max():.3e}")
    assert d_o.max() < 0.25 and d_l.max() < 0.5


def test_attend_mx_deterministic():
    w = mi.grad_slice()
    a, b = _mx_run(w), _mx_run(w)
    assert np.array_equal(a["O"].view(np.uint32), b["O"].view(np.uint32))
    assert np.array_equal(a["lse"].view(np.uint32), b["lse"].view(np.uint32))
