"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on the same seeded
inputs.

Bars: pooled means bit-exact; selections identical as sets except queries whose oracle k-th vs
(k+1)-th score gap is below 1e-4 relative (there the GPU's selection must still be legal and of
the right size, and the attention check below uses the GPU's selection); index inversion and
pair counts exact; outputs within max-abs 1e-4 (fp32) / 1e-2 (bf16) of the oracle, LSE likewise.
"""
import math
import os

import numpy as np
import pytest
import torch

import moc_inputs as mi
import parity_checks as pc
from oracle import moc_oracle as mo

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return torch.device("cuda:0")


def _moc():
    import sparse_chunk_routed_amd as moc
    return moc


_say = pc.say


class Run:
    """One workload through the GPU path, keeping host copies of every stage."""

    def __init__(self, w: mi.Workload, top_k=None, causal=None, p_max=None, lam=None):
        moc = _moc()
        dev = _dev()
        self.w = w
        self.top_k = w.top_k if top_k is None else top_k
        self.causal = w.causal if causal is None else causal
        self.p_max = w.p_max if p_max is None else p_max
        self.lam = w.lam if lam is None else lam
        _say(f"workload {w.name} L={w.L} C={w.C} B={w.B} H={w.H} d={w.d} {w.dtype} "
             f"k={self.top_k} causal={self.causal} p_max={self.p_max} lam={self.lam}")
        self.Q, self.K, self.V = mi.make_qkv(w)
        self.lay = moc.DeviceLayout.from_layout(w.layout, dev)
        self.cfg = moc.RouteCfg(self.top_k, self.causal, self.p_max, self.lam, w.max_drop_in, w.seed)
        Qd, Kd, Vd = (x.to(dev) for x in (self.Q, self.K, self.V))
        self.Qd, self.Kd, self.Vd = Qd, Kd, Vd
        self.kbar = moc.pool_keys(Kd, self.lay)
        self.sel, self.nsel = moc.route(Qd, self.kbar, self.lay, self.cfg)
        self.vl = moc.build_varlen(self.sel, self.nsel, self.lay, self.cfg, w.d, Qd.dtype)
        self.O, self.lse = moc.attend_fwd(Qd, Kd, Vd, self.lay, self.vl)
        torch.cuda.synchronize()
        self.h_kbar = self.kbar.cpu().numpy()
        self.h_sel = self.sel.cpu().numpy()
        self.h_nsel = self.nsel.cpu().numpy()
        self.h_O = self.O.float().cpu().numpy()
        self.h_lse = self.lse.cpu().numpy()
        self.h_pairs = self.vl.pair_count.cpu().numpy()
        _say("gpu path done")


def _check_selection(run: Run, o_route, kb, rows=None, label=None):
    """Selections against the oracle's (tie exemption, bounded and checked; see
    parity_checks.check_selection); returns the number of flagged queries that differ."""
    return pc.check_selection(run.w.layout, run.h_sel, run.h_nsel, o_route.sel, o_route.nsel,
                              o_route, run.Q, kb, run.causal, rows=rows,
                              label=label or run.w.name)


def _attend_rows(run: Run, rows, tol):
    O, lse = mo.attend(run.Q, run.K, run.V, run.w.layout, run.h_sel, rows=rows)
    got = np.stack([run.h_O[b, h, t] for (b, h, t) in rows])
    gl = np.array([run.h_lse[b, h, t] for (b, h, t) in rows])
    err = np.max(np.abs(got - O))
    lerr = np.max(np.abs(gl - lse))
    _say(f"attention rows={len(rows)} max|dO|={err:.3e} max|dlse|={lerr:.3e}")
    assert err <= tol, err
    assert lerr <= tol, lerr


def _sample_rows(w: mi.Workload, n_per_head: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    off = w.layout.chunk_offsets
    edges = set([0, w.L - 1])
    for c in range(w.C):
        edges.update([int(off[c]), int(off[c + 1]) - 1])
    rows = []
    for b in range(w.B):
        for h in range(w.H):
            ts = set(rng.choice(w.L, size=min(n_per_head, w.L), replace=False).tolist())
            ts.update(e for e in edges if rng.random() < 0.25)
            rows += [(b, h, int(t)) for t in sorted(ts)]
    return rows


# ----------------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny_run():
    return Run(mi.tiny())


def test_pool_bit_exact_tiny(tiny_run):
    ref = mo.pool_keys(tiny_run.K, tiny_run.w.layout)
    assert np.array_equal(tiny_run.h_kbar.view(np.uint32), ref.view(np.uint32))


def test_route_tiny(tiny_run):
    kb = mo.pool_keys(tiny_run.K, tiny_run.w.layout)
    r = mo.route(tiny_run.Q, kb, tiny_run.w.layout, tiny_run.top_k, tiny_run.causal)
    _check_selection(tiny_run, r, kb)
    mo.check_routing(tiny_run.w.layout, tiny_run.h_sel, tiny_run.h_nsel, tiny_run.top_k,
                     tiny_run.causal)


def _expected_buckets(sel, nsel, C):
    B, H, L, S = sel.shape
    buckets = {}
    for b in range(B):
        for h in range(H):
            for c in range(C):
                buckets[(b, h, c)] = []
            for t in range(L):
                for j in range(nsel[b, h, t]):
                    buckets[(b, h, int(sel[b, h, t, j]))].append(t)
    return buckets


def test_varlen_tiny(tiny_run):
    run = tiny_run
    w = run.w
    B, H, L = run.h_nsel.shape
    bo = run.vl.bucket_off().cpu().numpy()
    total = int(bo[-1])
    assert total == int(run.h_nsel.sum())
    bq = run.vl.bucket_q(total).cpu().numpy()
    slot = run.vl.slot(L).cpu().numpy()
    exp = _expected_buckets(run.h_sel, run.h_nsel, w.C)
    for (b, h, c), ts in exp.items():
        i = (b * H + h) * w.C + c
        assert list(bq[bo[i]:bo[i + 1]]) == ts, (b, h, c)
    # slot j of query t points at t inside bucket sel[t, j]
    for b in range(B):
        for h in range(H):
            for t in range(0, L, 7):
                for j in range(run.h_sel.shape[-1]):
                    if j < run.h_nsel[b, h, t]:
                        c = int(run.h_sel[b, h, t, j])
                        i = (b * H + h) * w.C + c
                        assert bo[i] <= slot[b, h, t, j] < bo[i + 1]
                        assert bq[slot[b, h, t, j]] == t
                    else:
                        assert slot[b, h, t, j] == -1
    ref = mo.pair_counts(w.layout, run.h_sel)
    assert np.array_equal(run.h_pairs, ref)
    assert int(run.h_pairs[0, 0]) == 6_307_840  # closed form for this layout (k=2, causal)
    bm = run.vl.struct.tile_rows
    assert run.vl.n_atiles() == math.ceil(128 / bm) + 4 * math.ceil(1024 / bm)


def test_attend_tiny_full(tiny_run):
    run = tiny_run
    O, lse = mo.attend(run.Q, run.K, run.V, run.w.layout, run.h_sel)
    err = np.max(np.abs(run.h_O - O))
    lerr = np.max(np.abs(run.h_lse - lse))
    _say(f"tiny full: max|dO|={err:.3e} max|dlse|={lerr:.3e}")
    assert err <= TOL["f32"] and lerr <= TOL["f32"]


def test_dense_equivalence_tiny():
    """top_k = all chunks, no causal mask: every query attends every key."""
    w = mi.tiny()
    run = Run(w, top_k=w.C, causal=False)
    assert int(run.h_pairs[0, 0]) == w.L * w.L
    Q = run.Q.double().numpy()[0]
    K = run.K.double().numpy()[0]
    V = run.V.double().numpy()[0]
    for h in range(w.H):
        s = Q[h] @ K[h].T / math.sqrt(w.d)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        Od = (p / p.sum(axis=1, keepdims=True)) @ V[h]
        err = np.max(np.abs(run.h_O[0, h] - Od))
        _say(f"dense head {h}: max|dO|={err:.3e}")
        assert err <= TOL["f32"]


@pytest.mark.parametrize("seed", range(8))
def test_random_layouts(seed):
    """Irregular chunk sizes, text first/last/absent, frame-is-shot, B=2, both head sizes,
    both dtypes, causal on/off, k from 0 to all."""
    rng = np.random.default_rng(1000 + seed)
    lay = mi.make_random_layout(rng, max_shots=5, max_frames=4, max_chunk=300,
                                frame_is_shot=seed in (3, 7))
    dtype = "bf16" if seed % 2 else "f32"
    d = 128 if seed in (1, 2, 5, 6) else 64
    top_k = min(lay.C, [0, 1, 3, lay.C, 2, 5, lay.C - 1, 4][seed])
    w = mi.Workload(f"rand{seed}", 2, 2, d, dtype, lay, top_k=top_k,
                    causal=seed not in (2, 6), clustered_keys=bool(seed % 2), seed=seed)
    run = Run(w)
    kb = mo.pool_keys(run.K, lay)
    assert np.array_equal(run.h_kbar.view(np.uint32), kb.view(np.uint32))
    r = mo.route(run.Q, kb, lay, top_k, w.causal)
    _check_selection(run, r, kb)
    mo.check_routing(lay, run.h_sel, run.h_nsel, top_k, w.causal)
    assert np.array_equal(run.h_pairs, mo.pair_counts(lay, run.h_sel))
    O, lse = mo.attend(run.Q, run.K, run.V, lay, run.h_sel)
    err = np.max(np.abs(run.h_O - O))
    lerr = np.max(np.abs(run.h_lse - lse))
    _say(f"rand{seed}: L={lay.L} C={lay.C} max|dO|={err:.3e} max|dlse|={lerr:.3e}")
    assert err <= TOL[dtype] and lerr <= TOL[dtype]


def test_determinism_tiny(tiny_run):
    again = Run(tiny_run.w)
    assert np.array_equal(again.h_sel, tiny_run.h_sel)
    assert np.array_equal(again.h_O.view(np.uint32), tiny_run.h_O.view(np.uint32))
    assert np.array_equal(again.h_lse.view(np.uint32), tiny_run.h_lse.view(np.uint32))


@pytest.mark.parametrize("name", ["short", "mid", "headline"])
def test_full_size_sampled(name):
    """Full-size workloads, the launch configuration the benchmark times: pooled means
    bit-exact everywhere, selections everywhere (tie exemption), pair counts exact, attention
    on sampled rows (every head, random rows plus chunk edges)."""
    w = mi.WORKLOADS[name]()
    run = Run(w)
    kb = mo.pool_keys(run.K, w.layout)
    assert np.array_equal(run.h_kbar.view(np.uint32), kb.view(np.uint32))
    _say("pool bit-exact")
    r = mo.route(run.Q, kb, w.layout, w.top_k, w.causal)
    _check_selection(run, r, kb)
    pc.check_legal(w.layout, run.h_sel, run.h_nsel, w.top_k, w.causal)
    _say("every selection legal")
    assert np.array_equal(run.h_pairs, mo.pair_counts(w.layout, run.h_sel))
    rows = _sample_rows(w, 24)
    _attend_rows(run, rows, TOL[w.dtype])
