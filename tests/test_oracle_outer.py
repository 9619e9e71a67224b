"""Pins of the oracle's outer-loop context routing (Mixture of Contexts summary, Appendix I):
coarse top-M segment selection by mean-pooled features, then inner routing restricted to the
query's own segment and the picked ones. CPU only."""
import numpy as np
import pytest

import moc_inputs as mi
from oracle import moc_oracle as mo

# small layout: 16 text tokens, 4 shots x 3 frames x 12 tokens (C = 13)
LAY = mi.build_layout(16, [3, 3, 3, 3], 12)
# segments: text | shot 0 | shot 1 frames 0-1 | shot 1 frame 2 + shot 2 | shot 3
SEGS = [0, 1, 4, 6, 10, 13]


def _rand(seed, d=8, B=1, H=2):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H, LAY.L, d)).astype(np.float32)
    K = rng.standard_normal((B, H, LAY.L, d)).astype(np.float32)
    return Q, K


def test_segments_derive_and_validate():
    G = mo.derive_segments(LAY, SEGS)
    assert G.nseg == 5
    assert list(G.is_text) == [True, False, False, False, False]
    assert list(G.tok_off) == [0, 16, 52, 76, 124, 160]
    with pytest.raises(ValueError):
        mo.derive_segments(LAY, [0, 2, 13])      # text chunk 0 and video chunk 1 together
    with pytest.raises(ValueError):
        mo.derive_segments(LAY, [0, 1, 1, 13])   # empty segment
    with pytest.raises(ValueError):
        mo.derive_segments(LAY, [0, 1, 12])      # does not end at C


def test_outer_constructed_case():
    """Keys constant per segment, v_s = s * e0 (text: 0); every query e0. The score of segment s
    is then s for every query segment, so by hand: causal top-1 of segment sq is sq - 1 (for
    sq >= 2), and non-causal top-2 of segment 1 is {3, 4}."""
    d = 4
    G = mo.derive_segments(LAY, SEGS)
    K = np.zeros((1, 1, LAY.L, d), dtype=np.float32)
    for s in range(G.nseg):
        K[0, 0, G.tok_off[s]:G.tok_off[s + 1], 0] = 0.0 if G.is_text[s] else float(s)
    Q = np.zeros_like(K)
    Q[..., 0] = 1.0
    r = mo.route_outer(Q, K, LAY, SEGS, 1, causal=True)
    assert r.seg_nsel[0, 0].tolist() == [0, 0, 1, 1, 1]
    assert r.seg_sel[0, 0, :, 0].tolist() == [-1, -1, 1, 2, 3]
    r2 = mo.route_outer(Q, K, LAY, SEGS, 2, causal=False)
    assert sorted(r2.seg_sel[0, 0, 1].tolist()) == [3, 4]
    assert r2.seg_sel[0, 0, 4].tolist() == [2, 3]
    # the text segment is never picked, and a segment never picks itself
    assert not np.any(r2.seg_sel == 0)
    for sq in range(G.nseg):
        assert sq not in r2.seg_sel[0, 0, sq].tolist()


def test_segment_features_are_size_weighted_chunk_means():
    """The mean over a segment equals the token-count-weighted average of its chunk means
    (computed here in binary64 from the chunk pooling; agreement to binary32 rounding)."""
    Q, K = _rand(1)
    r = mo.route_outer(Q, K, LAY, SEGS, 1, causal=True)
    G = mo.derive_segments(LAY, SEGS)
    D = mo.derive(LAY)
    for X, feat in ((Q, r.qseg), (K, r.kseg)):
        cm = mo.pool_keys(X, LAY).astype(np.float64)
        for s in range(G.nseg):
            cs = range(G.chunk_off[s], G.chunk_off[s + 1])
            w = np.array([D.sizes[c] for c in cs], dtype=np.float64)
            ref = np.tensordot(w, cm[:, :, list(cs), :], axes=([0], [2])) / w.sum()
            np.testing.assert_allclose(feat[:, :, s, :], ref, rtol=2e-6, atol=2e-7)


def test_outer_bruteforce_plain_loops():
    """Coarse selection recomputed with plain loops over segment pairs (np.mean features,
    explicit candidate filter, sort by (-score, id))."""
    for seed, M, causal in ((3, 1, True), (4, 2, True), (5, 2, False), (6, 3, False)):
        Q, K = _rand(seed, d=6, H=3)
        r = mo.route_outer(Q, K, LAY, SEGS, M, causal)
        G = mo.derive_segments(LAY, SEGS)
        for h in range(3):
            for sq in range(G.nseg):
                a, b = G.tok_off[sq], G.tok_off[sq + 1]
                q = Q[0, h, a:b].astype(np.float64).mean(axis=0).astype(np.float32)
                cands = []
                for s in range(G.nseg):
                    if G.is_text[s] or s == sq or (causal and s >= sq):
                        continue
                    ks = K[0, h, G.tok_off[s]:G.tok_off[s + 1]].astype(np.float64)
                    kf = ks.mean(axis=0).astype(np.float32)
                    cands.append((-float(np.dot(q.astype(np.float64), kf.astype(np.float64))), s))
                cands.sort()
                want = sorted(s for _, s in cands[:M])
                got = r.seg_sel[0, h, sq, :r.seg_nsel[0, h, sq]].tolist()
                if not r.gap_exempt[0, h, sq]:
                    assert got == want, (seed, h, sq, got, want)
                assert len(got) == min(M, len(cands))


def test_outer_mask_covers_own_and_picked_segments():
    Q, K = _rand(7)
    r = mo.route_outer(Q, K, LAY, SEGS, 1, causal=True)
    G = mo.derive_segments(LAY, SEGS)
    for h in range(2):
        for cq in range(LAY.C):
            sq = G.seg_of_chunk[cq]
            picked = set(r.seg_sel[0, h, sq, :r.seg_nsel[0, h, sq]].tolist()) | {sq}
            want = [G.seg_of_chunk[c] in picked for c in range(LAY.C)]
            assert r.cand_mask[0, h, cq].tolist() == want


def test_outer_with_every_segment_reduces_to_plain_routing():
    """M >= the number of segments: the mask admits every candidate, so inner routing equals
    ordinary MoC routing exactly."""
    Q, K = _rand(8)
    kb = mo.pool_keys(K, LAY)
    for causal in (True, False):
        r = mo.route_outer(Q, K, LAY, SEGS, len(SEGS), causal)
        plain = mo.route(Q, kb, LAY, 2, causal)
        inner = mo.route(Q, kb, LAY, 2, causal, cand_mask=r.cand_mask)
        assert np.array_equal(plain.sel, inner.sel) and np.array_equal(plain.nsel, inner.nsel)


def test_outer_zero_keeps_inner_routing_in_own_segment():
    Q, K = _rand(9)
    kb = mo.pool_keys(K, LAY)
    G = mo.derive_segments(LAY, SEGS)
    D = mo.derive(LAY)
    r = mo.route_outer(Q, K, LAY, SEGS, 0, causal=False)
    inner = mo.route(Q, kb, LAY, 3, False, cand_mask=r.cand_mask)
    mo.check_routing(LAY, inner.sel, inner.nsel, 3, False, cand_mask=r.cand_mask)
    for h in range(2):
        for t in range(LAY.L):
            sq = G.seg_of_chunk[D.chunk_of[t]]
            for c in inner.sel[0, h, t, :inner.nsel[0, h, t]]:
                assert G.seg_of_chunk[c] == sq


def test_outer_inner_routing_and_drop_in_respect_the_mask():
    Q, K = _rand(10)
    kb = mo.pool_keys(K, LAY)
    r = mo.route_outer(Q, K, LAY, SEGS, 1, causal=True)
    inner = mo.route(Q, kb, LAY, 2, True, cand_mask=r.cand_mask)
    mo.check_routing(LAY, inner.sel, inner.nsel, 2, True, cand_mask=r.cand_mask)
    sel, nsel = mo.drop_noise(inner, LAY, True, 0.3, 2.0, 8, seed=11, cand_mask=r.cand_mask)
    D = mo.derive(LAY)
    for h in range(2):
        for t in range(LAY.L):
            cq = D.chunk_of[t]
            for c in sel[0, h, t, :nsel[0, h, t]]:
                assert r.cand_mask[0, h, cq, c]
    # the restriction bites: some query has fewer candidates than without it
    masked = sum(len(mo.candidates(D, cq, True)) for cq in range(LAY.C))
    kept = sum(int(r.cand_mask[0, 0, cq, mo.candidates(D, cq, True)].sum())
               for cq in range(LAY.C) if len(mo.candidates(D, cq, True)))
    assert kept < masked
