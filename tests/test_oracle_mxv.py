"""Pins of the oracle's quantised values: V in MXFP8 with its 32-element blocks along the key
axis (mx_quantize_keys), attention over dequantised Q, K and V (attend_mxv), and the bound on
the error of rounding the softmax weights to e4m3 (pv_fp8_bound). CPU only."""
import math

import numpy as np

import moc_inputs as mi
from oracle import moc_oracle as mo

E4M3 = mo.e4m3_table()


def test_key_blocks_follow_the_key_axis():
    """One outlier moves the scale of exactly one block: its own (dim, 32-key block)."""
    L, d = 70, 64
    V = np.ones((1, 1, L, d))
    V[0, 0, 40, 5] = 1000.0
    codes, scales = mo.mx_quantize_keys(V)
    assert codes.shape == (1, 1, d, 96) and scales.shape == (1, 1, d, 3)
    # 1.0 -> E = -8 (code 119), element 1.0 * 2^8 = 256 = code 0x78
    want = np.full((d, 3), 119)
    want[5, 1] = 127 + 9 - 8          # floor(log2 1000) = 9
    assert np.array_equal(scales[0, 0], want)
    assert np.all(codes[0, 0, :, :L][np.arange(d) != 5] == 0x78)
    col = codes[0, 0, 5]
    assert np.all(col[:32] == 0x78) and np.all(col[64:L] == 0x78)
    assert col[40] == 0x7e                              # 1000 / 2 = 500 saturates to 448
    assert np.all(col[32:64][np.arange(32) != 8] == 0x30)   # 1.0 / 2 = 0.5
    assert np.all(codes[0, 0, :, L:] == 0)             # padding keys


def test_padding_keys_do_not_set_the_scale():
    V = np.zeros((1, 2, 33, 32))
    V[0, 0, 32, :] = 3.0          # the only real key of the second block
    V[0, 1, 32, :] = -0.01
    _, scales = mo.mx_quantize_keys(V)
    assert np.all(scales[0, 0, :, 1] == 127 + 1 - 8)
    assert np.all(scales[0, 1, :, 1] == 127 + math.floor(math.log2(0.01)) - 8)
    assert np.all(scales[0, :, :, 0] == 0)     # all-zero first blocks: E = -127


def test_representable_values_round_trip():
    """Values that are code * 2^E with a block maximum in [256, 448] come back unchanged."""
    rng = np.random.default_rng(3)
    L, d = 96, 32
    finite = np.array([c for c in range(256) if not math.isnan(E4M3[c])])
    big = np.array([c for c in range(127) if 256.0 <= E4M3[c] <= 448.0])
    codes = rng.choice(finite, size=(d, L)).astype(np.uint8)
    E = rng.integers(-20, 10, size=(d, L // 32))
    for i in range(d):
        for j in range(L // 32):
            codes[i, 32 * j + int(rng.integers(0, 32))] = rng.choice(big)
    cols = E4M3[codes] * np.repeat(2.0 ** E, 32, axis=1)
    V = cols.T[None, None]
    c2, s2 = mo.mx_quantize_keys(V)
    back = mo.mx_dequantize_keys(c2, s2, L)
    assert np.array_equal(back, V)
    assert np.array_equal(s2[0, 0], (E + 127).astype(np.uint8))


def _omega(lay: mi.Layout, t: int, sel_row) -> np.ndarray:
    """Text tokens, the query's own shot and the routed chunks, from the layout tables."""
    off, shot = lay.chunk_offsets, lay.chunk_shot
    c_t = int(np.searchsorted(off, t, side="right") - 1)
    keep = set(range(lay.text_begin, lay.text_end))
    for c in range(lay.C):
        if shot[c] >= 0 and shot[c] == shot[c_t]:
            keep.update(range(off[c], off[c + 1]))
    for c in sel_row:
        if c >= 0:
            keep.update(range(off[c], off[c + 1]))
    return np.array(sorted(keep))


def test_zero_queries_average_the_dequantised_values():
    """Q = 0 makes every weight equal: O is the plain mean of V' over Omega(t)."""
    w = mi.tiny()
    Q, K, V = mi.make_qkv(w)
    Q = np.zeros(Q.shape)
    rng = np.random.default_rng(5)
    sel = np.full((1, 2, w.L, 2), -1)
    for t in range(0, w.L, 97):
        sel[0, :, t, 0] = rng.integers(1, w.C)
    rows = [(0, h, t) for h in range(2) for t in range(0, w.L, 97)]
    O, _ = mo.attend_mxv(Q, K, V, w.layout, sel, rows=rows)
    Vd = mo.mx_dequantize_keys(*mo.mx_quantize_keys(V), w.L)
    for i, (b, h, t) in enumerate(rows):
        keys = _omega(w.layout, t, sel[b, h, t])
        assert np.allclose(O[i], Vd[b, h, keys].mean(axis=0), rtol=0, atol=1e-12)


def test_attend_mxv_is_attend_on_representable_inputs():
    w = mi.tiny()
    Q, K, V = mi.make_qkv(w)
    Qd = mo.mx_dequantize(*mo.mx_quantize(Q))
    Kd = mo.mx_dequantize(*mo.mx_quantize(K))
    Vd = mo.mx_dequantize_keys(*mo.mx_quantize_keys(V), w.L)
    sel = np.full((1, 2, w.L, 1), -1)
    rows = [(0, h, t) for h in range(2) for t in range(0, w.L, 211)]
    a, la = mo.attend_mxv(Qd, Kd, Vd, w.layout, sel, rows=rows)
    b, lb = mo.attend(Qd, Kd, Vd, w.layout, sel, rows=rows)
    assert np.allclose(a, b, rtol=0, atol=1e-13) and np.allclose(la, lb, rtol=0, atol=1e-13)


def _e4m3_round_value(x: np.ndarray) -> np.ndarray:
    return E4M3[mo.e4m3_round(x)]


def _simulated_row(x: np.ndarray, Vk: np.ndarray, delta: float, parts=None):
    """A kernel's P.V of one row with e4m3 weights: each part (a split of the keys) keeps its
    weights as 2^delta exp(x - max of the part), rounds them, divides by the part's unrounded
    sum; the parts are merged with their softmax weights."""
    if parts is None:
        parts = [np.arange(len(x))]
    num, den = 0.0, 0.0
    M = np.max(x)
    for idx in parts:
        xm = np.max(x[idx])
        wgt = 2.0 ** delta * np.exp(x[idx] - xm)
        o_part = (_e4m3_round_value(wgt) @ Vk[idx]) / np.sum(wgt)
        z = np.sum(np.exp(x[idx] - M))
        num = num + z * o_part
        den += z
    return num / den


def _bound_rows(Q, K, V, lay, sel, rows):
    return mo.pv_fp8_bound(Q, K, V, lay, sel, rows)


def test_fp8_weight_bound_holds_and_needs_both_terms():
    """The bound covers a brute-force e4m3 rounding of the weights at several running-max lags
    and splits; without its subnormal term it fails on a row whose weights are mostly tiny."""
    w = mi.tiny()
    Q, K, V = mi.make_qkv(w)
    Q, K, V = (mo._as_f64(x) for x in (Q, K, V))
    sel = np.full((1, 2, w.L, 2), -1)
    sel[0, :, :, 0] = 3
    rows = [(0, h, t) for h in range(2) for t in range(0, w.L, 53)]
    bound = _bound_rows(Q, K, V, w.layout, sel, rows)
    D = mo.derive(w.layout)
    scale = 1.0 / math.sqrt(w.d)
    worst = 0.0
    for i, (b, h, t) in enumerate(rows):
        keys = mo.key_set(D, t, sel[b, h, t])
        x = (K[b, h][keys] @ Q[b, h, t]) * scale
        p = np.exp(x - x.max())
        o = (p @ V[b, h][keys]) / p.sum()
        half = len(keys) // 2
        for delta in (0.0, 2.5, 8.0):
            for parts in (None, [np.arange(half), np.arange(half, len(keys))]):
                err = np.abs(_simulated_row(x, V[b, h][keys], delta, parts) - o)
                assert np.all(err <= bound[i] * (1 + 1e-9) + 1e-15)
                worst = max(worst, float(np.max(err / bound[i])))
    assert worst > 0.05   # the bound is not vacuous on these rows
    # one dominant key and many weights in the subnormal range of e4m3
    L = 4096
    lay = mi.layout_from_chunks([L], [0])
    x = np.full(L, math.log(2.0 ** -8.3))
    x[0] = 0.0
    q = np.zeros((1, 1, L, 1))
    q[0, 0, :, 0] = 1.0
    k = x.reshape(1, 1, L, 1)
    v = np.ones((1, 1, L, 1))
    rows = [(0, 0, 0)]
    full = mo.pv_fp8_bound(q, k, v, lay, np.full((1, 1, L, 1), -1), rows, scale=1.0)
    p = np.exp(x - x.max())
    err = abs(_simulated_row(x, v[0, 0], 0.0) - (p @ v[0, 0]) / p.sum())[0]
    assert err <= full[0, 0]
    assert err > 2.0 ** -4 * (p @ v[0, 0, :, 0]) / p.sum()   # the relative term alone is short
