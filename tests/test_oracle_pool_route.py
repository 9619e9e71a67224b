"""Pins of the oracle's pooling (mean-pooled chunk keys) and routing (candidates, top-k, causal
DAG). CPU only."""
from fractions import Fraction

import numpy as np
import pytest

import moc_inputs as mi
from oracle import moc_oracle as mo


def test_pool_constant_per_chunk_is_exact():
    lay = mi.build_layout(7, [3, 2], 11)
    B, H, d = 2, 3, 5
    const = np.random.default_rng(1).standard_normal((B, H, lay.C, d)).astype(np.float32)
    K = np.repeat(const, np.diff(lay.chunk_offsets), axis=2)
    kb = mo.pool_keys(K, lay)
    assert np.array_equal(kb, const)


def test_pool_dyadic_grid_matches_any_order_sum():
    """On multiples of 2^-8 in [-4, 4] every partial sum is exact, so the mean is
    RN32(RN64(sum)/n) whatever the summation order."""
    lay = mi.build_layout(9, [2, 3], 13)
    rng = np.random.default_rng(2)
    K = rng.integers(-1024, 1025, size=(1, 2, lay.L, 6)).astype(np.float64) / 256.0
    kb = mo.pool_keys(K, lay)
    off = lay.chunk_offsets
    for c in range(lay.C):
        n = off[c + 1] - off[c]
        ref = (K[:, :, off[c]:off[c + 1], :][:, :, ::-1, :].sum(axis=2) / n).astype(np.float32)
        assert np.array_equal(kb[:, :, c, :], ref)


def test_pool_matches_rational_mean_and_reduceat():
    """Random fp32 keys: equals the exactly rounded rational mean (brute force with
    fractions.Fraction, rounded once to binary64 and then to binary32), and np.add.reduceat's
    mean within 1 ulp of binary32."""
    lay = mi.build_layout(5, [2, 2], 9)
    K = np.random.default_rng(3).standard_normal((1, 1, lay.L, 4)).astype(np.float32)
    kb = mo.pool_keys(K, lay)
    off = lay.chunk_offsets
    for c in range(lay.C):
        n = int(off[c + 1] - off[c])
        for j in range(4):
            exact = sum(Fraction(float(x)) for x in K[0, 0, off[c]:off[c + 1], j])
            s64 = float(exact)  # correctly rounded to binary64
            assert kb[0, 0, c, j] == np.float32(s64 / n)
    red = (np.add.reduceat(K.astype(np.float64), off[:-1], axis=2)
           / np.diff(off)[None, None, :, None]).astype(np.float32)
    ulp = np.spacing(np.abs(red))
    assert np.all(np.abs(kb - red) <= ulp)


def _brute_topk(q, kb, D, cq, k, causal):
    cand = [c for c in range(D.C) if mo.allowed(D, cq, c, causal)]
    sc = {c: sum(float(a) * float(b) for a, b in zip(q, kb[c])) for c in cand}
    order = sorted(cand, key=lambda c: (-sc[c], c))
    return sorted(order[:min(k, len(cand))])


@pytest.mark.parametrize("causal", [True, False])
def test_route_matches_brute_force_on_tiny(causal):
    w = mi.tiny()
    lay = w.layout
    Q, K, V = mi.make_qkv(w)
    Qn, Kn = Q.numpy(), K.numpy()
    kb = mo.pool_keys(Kn, lay)
    r = mo.route(Qn, kb, lay, w.top_k, causal)
    D = mo.derive(lay)
    rng = np.random.default_rng(4)
    for t in rng.choice(lay.L, size=200, replace=False):
        for h in range(w.H):
            ref = _brute_topk(Qn[0, h, t], kb[0, h], D, int(D.chunk_of[t]), w.top_k, causal)
            if r.gap_exempt[0, h, t]:
                continue
            assert list(r.sel[0, h, t, :r.nsel[0, h, t]]) == ref
    mo.check_routing(lay, r.sel, r.nsel, w.top_k, causal)


def test_route_constructed_winner():
    """kbar_c = alpha_c * e_{c mod d} and q = e_j: among candidates, the score is alpha_c when
    c mod d == j and 0 otherwise, so the winners are known in advance."""
    d = 4
    lay = mi.build_layout(2, [1, 1, 1, 1, 1, 1], 3)  # text chunk 0, frames 1..6, one per shot
    C = lay.C
    alpha = np.array([0, 5, 7, 6, 1, 9, 2], dtype=np.float64)
    centres = np.zeros((1, 1, C, d))
    for c in range(1, C):
        centres[0, 0, c, c % d] = alpha[c]
    K = np.repeat(centres, np.diff(lay.chunk_offsets), axis=2)
    kb = mo.pool_keys(K, lay)
    L = lay.L
    Q = np.zeros((1, 1, L, d))
    last = lay.L - 1  # query in chunk 6 (shot 5): causal candidates are chunks 1..5
    for j in range(d):
        Q[0, 0, last, :] = 0
        Q[0, 0, last, j] = 1.0
        r = mo.route(Q, kb, lay, top_k=1, causal=True)
        cands = [c for c in range(1, 6)]
        best = max(cands, key=lambda c: (alpha[c] if c % d == j else 0.0, -c))
        assert list(r.sel[0, 0, last, :1]) == [best], j


def test_route_counts_and_predicate_random_layouts():
    for seed in range(8):
        rng = np.random.default_rng(50 + seed)
        lay = mi.make_random_layout(rng, max_shots=5, max_frames=3, max_chunk=9,
                                    frame_is_shot=bool(seed % 3 == 0))
        causal = bool(seed % 2)
        k = int(rng.integers(0, 5))
        Q = rng.standard_normal((1, 2, lay.L, 6))
        K = rng.standard_normal((1, 2, lay.L, 6))
        r = mo.route(Q, mo.pool_keys(K, lay), lay, k, causal)
        mo.check_routing(lay, r.sel, r.nsel, k, causal)


def test_causal_routing_graph_is_a_dag_and_noncausal_can_cycle():
    """Causal routing masks edges i->j with j >= i, so the routed chunk graph is acyclic
    (summary §3.2). Without it, two single-frame shots that can only pick each other form the
    2-cycle the pages describe (chunk 5 <-> chunk 6)."""
    w = mi.tiny()
    Q, K, V = mi.make_qkv(w)
    kb = mo.pool_keys(K.numpy(), w.layout)
    r = mo.route(Q.numpy(), kb, w.layout, w.top_k, True)
    E = mo.routed_edges(w.layout, r.sel)
    assert all(b < a for (a, b) in E)
    assert mo.is_dag(w.layout.C, E)
    lay = mi.build_layout(2, [1, 1], 3)
    rng = np.random.default_rng(6)
    Q = rng.standard_normal((1, 1, lay.L, 4))
    K = rng.standard_normal((1, 1, lay.L, 4))
    r2 = mo.route(Q, mo.pool_keys(K, lay), lay, 1, False)
    E2 = mo.routed_edges(lay, r2.sel)
    assert (1, 2) in E2 and (2, 1) in E2
    assert not mo.is_dag(lay.C, E2)
    r3 = mo.route(Q, mo.pool_keys(K, lay), lay, 1, True)
    assert mo.is_dag(lay.C, mo.routed_edges(lay, r3.sel))


def test_check_routing_rejects_broken_routings():
    lay = mi.build_layout(2, [2, 2], 3)
    rng = np.random.default_rng(7)
    Q = rng.standard_normal((1, 1, lay.L, 4))
    K = rng.standard_normal((1, 1, lay.L, 4))
    r = mo.route(Q, mo.pool_keys(K, lay), lay, 1, True)
    t = lay.L - 1  # last frame of shot 1; own-shot chunks 3,4 are mandatory, not candidates
    bad = r.sel.copy()
    bad[0, 0, t, 0] = 3
    with pytest.raises(AssertionError):
        mo.check_routing(lay, bad, r.nsel, 1, True)
    bad = r.sel.copy()
    bad[0, 0, t, 0] = 0  # text chunk
    with pytest.raises(AssertionError):
        mo.check_routing(lay, bad, r.nsel, 1, True)
    nbad = r.nsel.copy()
    nbad[0, 0, t] = 0
    with pytest.raises(AssertionError):
        mo.check_routing(lay, r.sel, nbad, 1, True)


def test_layout_validation():
    with pytest.raises(ValueError):
        mo.derive(mi.layout_from_chunks([3, 4, 5], [0, 1, 0]))  # shot 0 not contiguous
    lay = mi.build_layout(4, [2], 3)
    bad = mi.Layout(lay.chunk_offsets, lay.chunk_shot, 0, 3)  # text range cuts a chunk
    with pytest.raises(ValueError):
        mo.derive(bad)


# ---------------------------------------------------------------------------------------------
# The tie report of route(): gap_exempt marks a query whose k-th and (k+1)-th best candidate
# scores are closer than 1e-4 of the larger magnitude (the near-tie reading of the parity bar;
# an exact tie is decided by the lower chunk id). These pins build kbar from constant-per-chunk
# keys and a unit query, so every score is a chosen number.
# ---------------------------------------------------------------------------------------------

def _scored_route(scores, k, d=4):
    """Route one query placed after len(scores) single-frame shots whose chunk descriptors give
    the listed scores (chunk c+1 scores scores[c]); returns (routing, query token)."""
    n = len(scores)
    lay = mi.build_layout(2, [1] * (n + 1), 3, frame_is_shot=True)  # text, n frames, own frame
    kb = np.zeros((1, 1, lay.C, d), dtype=np.float64)
    for c, s in enumerate(scores):
        kb[0, 0, c + 1, 0] = s
    K = np.repeat(kb, np.diff(lay.chunk_offsets), axis=2)
    kbar = mo.pool_keys(K, lay)
    Q = np.zeros((1, 1, lay.L, d))
    t = lay.L - 1  # a query of the last frame: causal candidates are frames 1..n
    Q[0, 0, t, 0] = 1.0
    return mo.route(Q, kbar, lay, k, True), t


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_tie_report_band_edges(sign):
    """Gap of 0.5e-4 or 0.9e-4 relative: exempt; 1.1e-4 or 2e-4: not. Scores are placed out of
    chunk order; with sign = -1 the boundary pair is negative (the band is relative to the
    larger magnitude)."""
    for gap, want in ((0.5e-4, True), (2e-4, False), (0.9e-4, True), (1.1e-4, False)):
        if sign > 0:  # k = 2 best: chunk 2 (0.9), chunk 4 (0.5); then chunk 1 just below
            sc = [0.5 * (1.0 - gap), 0.9, 0.1, 0.5]
        else:         # k = 2 best: chunk 2 (-0.2), chunk 4 (-0.5); then chunk 1 just below
            sc = [-0.5 * (1.0 + gap), -0.2, -3.0, -0.5]
        r, t = _scored_route(sc, 2)
        s = np.sort(np.asarray(sc, dtype=np.float32).astype(np.float64))[::-1]
        rel = (s[1] - s[2]) / max(abs(s[1]), abs(s[2]))
        assert abs(rel - gap) < 1e-6  # the constructed gap survives rounding to binary32
        assert list(r.sel[0, 0, t, :2]) == [2, 4]
        assert bool(r.gap_exempt[0, 0, t]) is want, (gap, sign, rel)


def test_tie_report_exact_ties_and_few_candidates():
    # an exact tie at a non-zero score is inside the band; it is decided by the lower chunk id
    r, t = _scored_route([0.2, 0.7, 0.7, 0.1], 1)
    assert bool(r.gap_exempt[0, 0, t])
    assert list(r.sel[0, 0, t, :1]) == [2]
    # an exact tie at zero is not (the band is empty); the lower chunk id wins
    r, t = _scored_route([-0.2, 0.0, 0.0, -0.1], 1)
    assert not bool(r.gap_exempt[0, 0, t])
    assert list(r.sel[0, 0, t, :1]) == [2]
    # #candidates <= k: every candidate is taken, nothing is ever exempt, even with equal scores
    for k in (3, 4, 6):
        r, t = _scored_route([0.5, 0.5, 0.5], k)
        assert not bool(r.gap_exempt[0, 0, t])
        assert list(r.sel[0, 0, t, :r.nsel[0, 0, t]]) == [1, 2, 3]


def test_tie_report_compares_sorted_neighbours():
    """The flag compares the k-th and (k+1)-th of the sorted order, not neighbours in chunk
    order: two near-equal scores far from the k boundary leave the query not exempt."""
    r, t = _scored_route([0.40000, 0.99, 0.40001, 0.2, 0.7], 2)
    assert not bool(r.gap_exempt[0, 0, t])        # 0.7 vs 0.40001 at the boundary
    r, t = _scored_route([0.40000, 0.99, 0.40001, 0.2, 0.7], 3)
    assert bool(r.gap_exempt[0, 0, t])            # 0.40001 vs 0.40000 at the boundary


def test_tie_report_is_rare_on_seeded_workloads():
    """On the tiny workload and the gradient slice only a handful of queries carry the flag
    (measured: 1 of 8,448 and 5 of 50,688); a flag set too broadly would empty every selection
    check that skips flagged queries."""
    for w in (mi.tiny(), mi.grad_slice()):
        Q, K, V = mi.make_qkv(w)
        r = mo.route(Q, mo.pool_keys(K, w.layout), w.layout, w.top_k, w.causal)
        frac = float(r.gap_exempt.mean())
        assert frac < 1e-3, (w.name, frac)
