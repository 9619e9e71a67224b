"""Pins of pair counts (closed forms, page figures) and of the routing-noise generator
(published SplitMix64 vectors, Poisson CDF from scipy, sampling statistics, set relations)."""
import json
import math
import os

import numpy as np
import pytest

import moc_inputs as mi
from oracle import moc_oracle as mo
from oracle import rng as orng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _closed_form_pairs(n_txt, shot_frames, f, k):
    """Equal frames of f tokens, text first, causal, anchors = text + own shot:
    pairs = N_txt^2 + sum_s n_s (N_txt + n_s + min(k, F_<s) f)."""
    tot = n_txt * n_txt
    before = 0
    for nf in shot_frames:
        ns = nf * f
        tot += ns * (n_txt + ns + min(k, before) * f)
        before += nf
    return tot


def _oracle_pairs(w):
    """Route one head of the workload with the oracle and count pairs."""
    w1 = mi.Workload(w.name, 1, 1, w.d, w.dtype, w.layout, w.top_k, w.causal,
                     w.clustered_keys, seed=w.seed)
    Q, K, V = mi.make_qkv(w1)
    kb = mo.pool_keys(K, w.layout)
    r = mo.route(Q, kb, w.layout, w.top_k, w.causal)
    return int(mo.pair_counts(w.layout, r.sel)[0, 0])


def test_pairs_tiny_closed_form():
    w = mi.tiny()
    got = _oracle_pairs(w)
    assert got == _closed_form_pairs(128, [4] * 4, 256, 2) == 6_307_840
    assert abs((1 - got / w.L ** 2) - 0.6465) < 1e-4


@pytest.mark.slow
@pytest.mark.parametrize("name,frames,ntxt,k,expect", [
    ("mid", [8] * 8, 512, 4, 1_842_509_824),
    ("headline_uniform", [14] * 8, 512, 2, 4_382_589_184),
])
def test_pairs_large_closed_form(name, frames, ntxt, k, expect):
    w = mi.WORKLOADS[name]()
    got = _oracle_pairs(w)
    assert got == _closed_form_pairs(ntxt, frames, mi.FRAME_TOKENS, k) == expect


def test_pairs_short_single_shot_closed_form():
    """Each frame its own shot: anchors are text + own frame; causal candidates are earlier
    frames."""
    w = mi.short()
    n_txt, f, F = 256, mi.FRAME_TOKENS, 21
    expect = n_txt * n_txt + sum(f * (n_txt + f + min(3, i) * f) for i in range(F))
    assert expect == 198_272_896
    # routing does not change the count (every frame has at least min(k, i) candidates)
    lay = w.layout
    sel = np.full((1, 1, lay.L, 3), -1, dtype=np.int32)
    D = mo.derive(lay)
    for t in range(lay.L):
        c = int(D.chunk_of[t])
        cand = mo.candidates(D, c, True)
        sel[0, 0, t, :min(3, len(cand))] = cand[:3]
    assert int(mo.pair_counts(lay, sel)[0, 0]) == expect


@pytest.mark.slow
def test_headline_k_is_largest_with_85pct_pruned():
    """Table 1 of the pages: about 85% of query-key pairs pruned on ~180k-token 8-shot scenes.
    With the irregular 8-shot layouts (seeds 0-7), k=2 prunes >= 85% and k=3 does not."""
    for seed in range(8):
        w = mi.headline(seed)
        frames = mi.irregular_shot_frames(seed)
        p2 = _closed_form_pairs(512, frames, mi.FRAME_TOKENS, 2)
        p3 = _closed_form_pairs(512, frames, mi.FRAME_TOKENS, 3)
        assert 1 - p2 / w.L ** 2 >= 0.85
        assert 1 - p3 / w.L ** 2 < 0.85
    got = _oracle_pairs(mi.headline(0))
    assert got == _closed_form_pairs(512, mi.irregular_shot_frames(0), mi.FRAME_TOKENS, 2)


def test_page_figures_eq5_and_table1():
    g = json.load(open(os.path.join(GOLDEN, "moc_page_figures.json")))
    ex = g["eq5_example"]
    assert abs(mo.dense_flops(ex["L"], ex["d"]) - ex["dense_flops"]) / ex["dense_flops"] < 5e-3
    # Headline shape (8 shots of 14 frames, ~175k tokens): dense vs MoC attention FLOPs per
    # head land at the pages' 1.7e13 -> 2.3e12 at their ~180k tokens (2 significant digits,
    # our token count is 2.7% lower, so a 10% band).
    L = 512 + 112 * mi.FRAME_TOKENS
    pairs = _closed_form_pairs(512, [14] * 8, mi.FRAME_TOKENS, 2)
    t1 = g["table1"]
    assert abs(mo.dense_flops(L, 128) - t1["attention_flops_dense"]) / t1["attention_flops_dense"] < 0.1
    assert abs(mo.attention_flops(pairs, 128) - t1["attention_flops_moc"]) / t1["attention_flops_moc"] < 0.1
    assert 1 - pairs / L ** 2 >= t1["pruned_fraction"]


def test_splitmix64_published_vectors():
    g = json.load(open(os.path.join(GOLDEN, "splitmix64_vectors.json")))
    for v in g["vectors"]:
        outs = orng.splitmix64_stream(v["seed"], 3)
        if "outputs_hex" in v:
            assert outs == [int(x, 16) for x in v["outputs_hex"]]
        else:
            assert outs == [int(x) for x in v["outputs_dec"]]
    # H32 is the high word of stream output ctr+1
    assert orng.h32(1234567, 0) == 6457827717110365317 >> 32
    assert orng.h32(1234567, 2) == 9817491932198370423 >> 32


def test_poisson_thresholds_match_scipy_cdf():
    from scipy.stats import poisson
    for lam in (0.25, 1.0, 2.5):
        thr = orng.poisson_thresholds(lam, 8)
        for i in range(8):
            ref = poisson.cdf(i, lam) * 2 ** 32
            assert abs(thr[i] - ref) <= 2.0
        assert all(thr[i] <= thr[i + 1] for i in range(7))


def test_poisson_draw_histogram():
    """Chi-square of m over 1e5 counter words against Poisson(1) truncated at 8."""
    from scipy.stats import chi2, poisson
    thr = orng.poisson_thresholds(1.0, 8)
    n = 100_000
    cnt = np.zeros(9)
    for i in range(n):
        m = orng.poisson_from_word(orng.h32(99, i), thr, 8)
        cnt[m] += 1
    pr = np.array([poisson.pmf(i, 1.0) for i in range(8)] + [poisson.sf(7, 1.0)])
    # merge tail bins with small expectation
    exp = pr * n
    obs = cnt
    keep = exp >= 5
    stat = np.sum((obs[keep] - exp[keep]) ** 2 / exp[keep])
    tail_o, tail_e = obs[~keep].sum(), exp[~keep].sum()
    stat += (tail_o - tail_e) ** 2 / max(tail_e, 1e-9)
    dof = keep.sum()
    assert stat < chi2.ppf(0.999, dof)


def _noise_setup(k, seed=0):
    lay = mi.build_layout(4, [3, 3, 3, 2], 5)
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((1, 2, lay.L, 8))
    K = rng.standard_normal((1, 2, lay.L, 8))
    r = mo.route(Q, mo.pool_keys(K, lay), lay, k, True)
    return lay, r


def test_drop_noise_set_relations():
    """dropped subset of T; added subset of candidates minus T; anchors untouched;
    |sel| = |T| - nd + min(m, |pool|); the causal DAG survives."""
    k = 5
    lay, r = _noise_setup(k)
    D = mo.derive(lay)
    sel, nsel = mo.drop_noise(r, lay, True, 0.3, 1.0, 8, seed=17)
    thr = orng.poisson_thresholds(float(np.float32(1.0)), 8)
    B, H, L, S = sel.shape
    assert S == r.k_eff + 8
    for h in range(H):
        for t in range(L):
            T = set(int(c) for c in r.sel[0, h, t, :r.nsel[0, h, t]])
            out = [int(c) for c in sel[0, h, t, :nsel[0, h, t]]]
            assert out == sorted(set(out))
            cand = set(int(c) for c in mo.candidates(D, int(D.chunk_of[t]), True))
            kept = set(out) & T
            added = set(out) - T
            assert added <= cand - T
            # recompute the draw counts from the generator
            word = orng.h32(17, orng.counter(0, h, t, 0, 0, H, L))
            p = float(word >> 8) * 2.0 ** -24 * float(np.float32(0.3))
            nd = min(math.floor(p * r.k_eff), len(T))
            m = orng.poisson_from_word(orng.h32(17, orng.counter(0, h, t, 2, 0, H, L)), thr, 8)
            assert len(kept) == len(T) - nd
            assert len(added) == min(m, len(cand - T))
    assert mo.is_dag(lay.C, mo.routed_edges(lay, sel))


def test_drop_off_expectation():
    """E floor(p k) with p ~ U(0, 0.3): 0 for k <= 3, 1/6 for k = 4, 1/3 for k = 5."""
    for k, expect in ((3, 0.0), (4, 1 / 6), (5, 1 / 3)):
        n = 60_000
        tot = 0
        for i in range(n):
            u = float(orng.h32(5, orng.counter(0, 0, i, 0, 0, 1, n)) >> 8) * 2.0 ** -24
            tot += math.floor(u * float(np.float32(0.3)) * k)
        assert abs(tot / n - expect) < 0.01, (k, tot / n)


def test_drop_noise_reduces_to_identity_when_disabled():
    lay, r = _noise_setup(3)
    sel, nsel = mo.drop_noise(r, lay, True, 0.0, 0.0, 8, seed=1)
    assert np.array_equal(sel, r.sel) and np.array_equal(nsel, r.nsel)


def _pick_layout():
    """Text + 12 single-frame shots of 10,000 tokens: a query of the last frame has the 11
    earlier frames (chunks 1..11) as causal candidates, and there are 10,000 such queries."""
    lay = mi.build_layout(16, [1] * 12, 10_000, frame_is_shot=True)
    D = mo.derive(lay)
    ts = range(int(lay.chunk_offsets[-2]), int(lay.chunk_offsets[-1]))
    return lay, D, ts


def _chi2_uniform(counts):
    """Chi-square statistic and degrees of freedom of counts against a uniform law."""
    from scipy.stats import chi2
    c = np.asarray(list(counts.values()), dtype=np.float64)
    e = c.sum() / len(c)
    stat = float(np.sum((c - e) ** 2 / e))
    return stat, chi2.ppf(0.999, len(c) - 1)


def test_drop_off_picks_uniform_subsets():
    """Drop-off removes its floor(p k) chunks uniformly at random from the routed set ([MoC-S]
    §3.1, "at random"): given the number dropped, every subset of that size is equally likely.
    k = 4, p_max = 1 makes nd uniform on {0, 1, 2, 3}; over 1e5 queries (10 seeds x 10,000
    queries) each nd >= 1 gets a chi-square test over its C(4, nd) subsets."""
    from itertools import combinations
    lay, D, ts = _pick_layout()
    T = [1, 4, 7, 10]
    by_nd = {nd: {frozenset(s): 0 for s in combinations(T, nd)} for nd in (1, 2, 3)}
    n_nd = np.zeros(5)
    for seed in range(10):
        for t in ts:
            out = mo.drop_noise_row(D, T, 0, 0, t, 1, 4, True, 1.0, 0.0, 8, seed, None)
            dropped = frozenset(T) - frozenset(out)
            n_nd[len(dropped)] += 1
            if dropped:
                by_nd[len(dropped)][dropped] += 1
    assert n_nd[4] == 0
    assert np.all(np.abs(n_nd[:4] / n_nd.sum() - 0.25) < 0.01)  # floor(4 u) is uniform
    for nd, counts in by_nd.items():
        stat, lim = _chi2_uniform(counts)
        assert stat < lim, (nd, stat, lim, counts)


def test_drop_in_picks_uniform_subsets():
    """Drop-in adds min(m, |pool|) chunks uniformly at random from the candidates not already
    routed: given m, every m-subset of the pool is equally likely. T = {3, 8} leaves a pool of 9
    chunks; lambda = 2 puts about 27% of 1e5 queries at m = 1 and 27% at m = 2 (chi-square over
    9 and 36 subsets)."""
    lay, D, ts = _pick_layout()
    T = [3, 8]
    pool = [c for c in range(1, 12) if c not in T]
    thr = orng.poisson_thresholds(float(np.float32(2.0)), 8)
    counts = {1: {}, 2: {}}
    from itertools import combinations
    for m in (1, 2):
        counts[m] = {frozenset(s): 0 for s in combinations(pool, m)}
    for seed in range(10):
        for t in ts:
            out = mo.drop_noise_row(D, T, 0, 0, t, 1, 2, True, 0.0, 2.0, 8, seed, thr)
            added = frozenset(out) - frozenset(T)
            assert frozenset(T) <= frozenset(out) and added <= frozenset(pool)
            if len(added) in counts:
                counts[len(added)][added] += 1
    for m, c in counts.items():
        assert sum(c.values()) > 20_000
        stat, lim = _chi2_uniform(c)
        assert stat < lim, (m, stat, lim)


def test_drop_in_never_re_adds_dropped_chunks():
    """Drop-off then drop-in: the drop-in pool is the candidates minus the ORIGINAL routed set,
    so a dropped chunk never comes back in the same draw."""
    lay, D, ts = _pick_layout()
    T = [2, 5, 6, 9, 11]
    thr = orng.poisson_thresholds(float(np.float32(3.0)), 8)
    seen_drop = 0
    for t in list(ts)[:5000]:
        out = mo.drop_noise_row(D, T, 0, 0, t, 1, 5, True, 1.0, 3.0, 8, 3, thr)
        kept = set(out) & set(T)
        dropped = set(T) - kept
        seen_drop += bool(dropped)
        assert not (dropped & set(out))
    assert seen_drop > 3000
