"""Pins of the oracle's MXFP8 quantisation of Q and K (the quantised-scores variant): E4M3
element values (OCP OFP8), round-to-nearest-even with saturation, the MX shared block scale,
and attention over the dequantised values. CPU only."""
import json
import math
import os

import numpy as np
import pytest

import moc_inputs as mi
from oracle import moc_oracle as mo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_e4m3_blocks.json")


def test_golden_blocks_worked_by_hand():
    g = json.load(open(GOLDEN))
    for blk in g["blocks"]:
        x = np.zeros(32)
        x[:len(blk["x"])] = blk["x"]
        codes, scales = mo.mx_quantize(x[None, :])
        want = np.zeros(32, dtype=np.uint8)
        want[:len(blk["codes"])] = [int(c, 16) for c in blk["codes"]]
        assert codes[0].tolist() == want.tolist(), blk["note"]
        assert int(scales[0, 0]) == blk["scale"], blk["note"]


def test_e4m3_values_fixed_by_the_format():
    t = mo.e4m3_table()
    assert t[0x00] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9      # subnormals m/8 * 2^-6
    assert t[0x08] == 2.0 ** -6                                      # smallest normal
    assert t[0x38] == 1.0 and t[0x40] == 2.0 and t[0x3c] == 1.5
    assert t[0x7e] == 448.0 and t[0xfe] == -448.0                  # largest finite
    assert math.isnan(t[0x7f]) and math.isnan(t[0xff])
    assert np.sum(np.isnan(t)) == 2
    pos = t[:127]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(t[128:255], -t[:127])
    # spacing: 8 values per binade, step 2^(e-10) in binade [2^(e-7), 2^(e-6))
    for e in range(1, 15):
        b = pos[8 * e:8 * e + 8]
        assert np.allclose(np.diff(b), 2.0 ** (e - 10)) and b[0] == 2.0 ** (e - 7)


def _brute_round(v: float) -> int:
    """Nearest finite E4M3 value to the saturated |v| by scanning every code; ties to the even
    code; the sign bit from v."""
    a = min(abs(v), 448.0)
    best, bd = None, None
    for c in range(127):
        d = abs(mo.e4m3_value(c) - a)
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return best | (0x80 if math.copysign(1.0, v) < 0 else 0)


def test_rounding_against_brute_force():
    rng = np.random.default_rng(0)
    vals = list(rng.standard_normal(400) * 2.0 ** rng.integers(-12, 10, 400))
    t = mo.e4m3_table()
    for c in range(126):  # every midpoint and its neighbours, both signs
        m = (t[c] + t[c + 1]) / 2
        vals += [m, np.nextafter(m, 0), np.nextafter(m, 1e9), t[c]]
    vals += [448.0, 450.0, 464.0, 479.0, 1e6, 0.0, -0.0, 2.0 ** -10, 2.0 ** -11]
    vals += [-v for v in vals]
    got = mo.e4m3_round(np.array(vals))
    for v, g in zip(vals, got):
        assert int(g) == _brute_round(float(v)), (v, hex(int(g)))


def test_scale_rule_and_error_bounds():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((200, 64)) * 2.0 ** rng.integers(-30, 30, (200, 1))
    X[5, :32] = 0.0
    codes, scales = mo.mx_quantize(X)
    Y = mo.mx_dequantize(codes, scales)
    t = mo.e4m3_table()
    for r in range(X.shape[0]):
        for blk in range(2):
            x = X[r, 32 * blk:32 * blk + 32]
            amax = np.max(np.abs(x))
            E = int(scales[r, blk]) - 127
            if amax == 0:
                assert E == -127 and not codes[r, 32 * blk:32 * blk + 32].any()
                continue
            assert 256.0 <= amax / 2.0 ** E < 512.0          # the largest element lands in the top binade
            c = codes[r, 32 * blk:32 * blk + 32]
            assert ((c & 0x7f) >> 3).max() == 15             # exponent field of the largest element
            y = Y[r, 32 * blk:32 * blk + 32]
            big = np.abs(x) / 2.0 ** E >= 2.0 ** -6          # normal range: half-ulp relative bound
            sat = np.abs(x) / 2.0 ** E > 448.0
            assert np.all(np.abs(y - x)[big & ~sat] <= 2.0 ** -4 * np.abs(x)[big & ~sat])
            assert np.all(np.abs(y - x)[~big] <= 2.0 ** -10 * 2.0 ** E)
            assert np.all(np.abs(y[sat]) == 448.0 * 2.0 ** E)
            assert np.all(t[c] * 2.0 ** E == y)


def test_representable_values_round_trip():
    rng = np.random.default_rng(2)
    t = mo.e4m3_table()
    for _ in range(50):
        E = int(rng.integers(-120, 100))
        c = rng.integers(0, 127, 32).astype(np.uint8)
        c[int(rng.integers(0, 32))] = int(rng.integers(0x78, 0x7f))   # block max in [256, 448]
        c |= (rng.integers(0, 2, 32) << 7).astype(np.uint8)
        x = t[c] * 2.0 ** E
        codes, scales = mo.mx_quantize(x[None])
        assert int(scales[0, 0]) == E + 127
        assert np.array_equal(mo.mx_dequantize(codes, scales)[0], x)


def test_attend_mx_is_attend_on_representable_inputs():
    """When Q and K are already MXFP8 values, the quantised attention is the exact one."""
    w = mi.tiny()
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in mi.make_qkv(w)[:3])
    Qr = mo.mx_dequantize(*mo.mx_quantize(Q))
    Kr = mo.mx_dequantize(*mo.mx_quantize(K))
    kb = mo.pool_keys(K, w.layout)
    r = mo.route(Q, kb, w.layout, w.top_k, w.causal)
    O1, l1 = mo.attend_mx(Qr, Kr, V, w.layout, r.sel)
    O2, l2 = mo.attend(Qr, Kr, V, w.layout, r.sel)
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2)
    rows = [(0, 0, 3), (0, 1, 100), (0, 1, w.L - 1)]
    O3, l3 = mo.attend_mx(Q, K, V, w.layout, r.sel, rows=rows)
    O4, l4 = mo.attend_mx(Q, K, V, w.layout, r.sel)
    for i, (b, h, t) in enumerate(rows):
        assert np.array_equal(O3[i], O4[b, h, t]) and l3[i] == l4[b, h, t]


def test_quantisation_error_of_the_scores_is_bounded():
    """Each dequantised element is within 2^-4 relative (normal range) of the input, so a score
    q.k moves by at most 2^-4 (2 + 2^-4) sum |q_i k_i| plus the subnormal terms."""
    w = mi.tiny()
    Q, K = (np.asarray(x, dtype=np.float64) for x in mi.make_qkv(w)[:2])
    Qd = mo.mx_dequantize(*mo.mx_quantize(Q))
    Kd = mo.mx_dequantize(*mo.mx_quantize(K))
    q, k = Q[0, 0, :50], K[0, 0, :50]
    s = q @ k.T
    sd = Qd[0, 0, :50] @ Kd[0, 0, :50].T
    bound = (2.0 ** -4 * (2 + 2.0 ** -4)) * (np.abs(q) @ np.abs(k).T) + 1e-6
    assert np.all(np.abs(sd - s) <= bound)
    assert np.max(np.abs(sd - s)) > 0  # the quantisation is not the identity here
