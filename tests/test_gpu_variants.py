"""GPU parity of layout variants beyond the multi-shot workloads.

* Single-shot clips with fixed-size chunks that cut across frames, every chunk its own shot,
  non-causal routing with top-k 3 (Mixture of Contexts summary, Appendix E-G and Table 3: about
  6,300 tokens, chunk sizes 64 to 1,024): pooled means bit-exact, every selection (tie
  exemption), pair counts exact, attention on sampled rows, and the backward at chunk 256.
* Dense attention as a layout: one shot holding every token and no routing, which is the
  same-GPU dense baseline of the length sweep; checked against plain softmax attention, at
  small lengths in full and at the 8-shot length (175,232 tokens) on sampled rows.
* The longest layout of the length sweep, 24 shots of 14 frames (524,672 tokens): pooled means
  bit-exact, every selection, pair counts exact, attention on sampled rows.
"""
import math

import numpy as np
import pytest
import torch

import moc_inputs as mi
import parity_checks as pc
from oracle import moc_oracle as mo
from test_gpu_parity import TOL, Run, _attend_rows, _check_selection, _sample_rows, _say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("chunk", [64, 128, 256, 512, 1024])
def test_single_shot_fixed_chunks(chunk):
    w = mi.single_shot(chunk=chunk)
    assert w.L == 6304 and not w.causal and w.top_k == 3
    run = Run(w)
    kb = mo.pool_keys(run.K, w.layout)
    assert np.array_equal(run.h_kbar.view(np.uint32), kb.view(np.uint32))
    r = mo.route(run.Q, kb, w.layout, w.top_k, w.causal)
    _check_selection(run, r, kb)
    mo.check_routing(w.layout, run.h_sel, run.h_nsel, w.top_k, w.causal)
    assert np.array_equal(run.h_pairs, mo.pair_counts(w.layout, run.h_sel))
    _attend_rows(run, _sample_rows(w, 40, seed=chunk), TOL[w.dtype])


def test_single_shot_backward_c256():
    """Backward on the chunk-256 single-shot layout (two heads, all rows) against the oracle's
    fp64 backward over the GPU's routed sets."""
    import sparse_chunk_routed_amd as moc
    w = mi.single_shot(chunk=256, H=2)
    dev = torch.device("cuda:0")
    Q, K, V, dO = mi.make_qkv(w, with_dout=True)
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    cfg = moc.RouteCfg(w.top_k, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed)
    Qd, Kd, Vd, dOd = (x.to(dev) for x in (Q, K, V, dO))
    r = moc.forward(Qd, Kd, Vd, lay, cfg)
    dQ, dK, dV = moc.attend_bwd(Qd, Kd, Vd, r.O, r.lse, dOd, lay, r.varlen)
    torch.cuda.synchronize()
    sel = r.sel.cpu().numpy()
    ref = mo.attend_bwd(Q, K, V, dO, w.layout, sel)
    for name, a, b in (("dQ", dQ, ref[0]), ("dK", dK, ref[1]), ("dV", dV, ref[2])):
        err = float(np.max(np.abs(a.float().cpu().numpy() - b)))
        _say(f"c256 backward {name}: max|err|={err:.3e} (max|ref|={np.max(np.abs(b)):.3e})")
        assert err <= TOL["bf16"], (name, err)


@pytest.mark.parametrize("L", [1000, 4321])
def test_dense_layout(L):
    """One shot holding every token, no text, top_k 0: plain bidirectional softmax attention."""
    sizes = [L // 3, L // 3, L - 2 * (L // 3)]
    lay = mi.layout_from_chunks(sizes, [0, 0, 0])
    w = mi.Workload(f"dense_L{L}", 1, 2, 128, "bf16", lay, top_k=0, causal=True,
                    clustered_keys=True, seed=7)
    run = Run(w)
    assert int(run.h_pairs[0, 0]) == L * L
    Q = run.Q.double().numpy()[0]
    K = run.K.double().numpy()[0]
    V = run.V.double().numpy()[0]
    for h in range(w.H):
        s = Q[h] @ K[h].T / math.sqrt(w.d)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        Od = (p / p.sum(axis=1, keepdims=True)) @ V[h]
        lse = (m[:, 0] + np.log(p.sum(axis=1)))
        err = np.max(np.abs(run.h_O[0, h] - Od))
        lerr = np.max(np.abs(run.h_lse[0, h] - lse))
        _say(f"dense L={L} head {h}: max|dO|={err:.3e} max|dlse|={lerr:.3e}")
        assert err <= TOL["bf16"] and lerr <= TOL["bf16"]


def test_dense_layout_8_shot_length_sampled():
    """The length sweep's dense baseline at 8 shots: one shot of 175,232 tokens, no routing, so
    every query attends every key. Sampled rows of every head against plain softmax attention
    (the oracle's key set is the whole sequence)."""
    w = mi.dense(n_shots=8)
    run = Run(w)
    assert int(run.h_pairs.sum()) == w.B * w.H * w.L * w.L
    rng = np.random.default_rng(3)
    rows = [(0, h, int(t)) for h in range(w.H)
            for t in list(rng.choice(w.L, 3, replace=False)) + [0, w.L - 1]]
    _attend_rows(run, rows, TOL[w.dtype])


@pytest.mark.parametrize("n_shots,L,C", [(16, 349_952, 225), (24, 524_672, 337)])
def test_shots_sweep_sampled(n_shots, L, C):
    """The two longest layouts of the length sweep (512 text + n shots x 14 frames x 1,560
    tokens: 349,952 tokens at 16 shots, 524,672 at 24; top-k 2): pooled means bit-exact for every
    head and chunk, every selection against the oracle (tie exemption, legality), pair counts
    exact, and attention on sampled rows and chunk edges of every head."""
    w = mi.shots(n_shots=n_shots)
    assert w.L == L and w.C == C
    run = Run(w)
    kb = mo.pool_keys(run.K, w.layout)
    assert np.array_equal(run.h_kbar.view(np.uint32), kb.view(np.uint32))
    _say("pool bit-exact")
    r = mo.route(run.Q, kb, w.layout, w.top_k, w.causal)
    _check_selection(run, r, kb)
    pc.check_legal(w.layout, run.h_sel, run.h_nsel, w.top_k, w.causal)
    assert np.array_equal(run.h_pairs, mo.pair_counts(w.layout, run.h_sel))
    _say(f"pairs {int(run.h_pairs.sum())} exact")
    _attend_rows(run, _sample_rows(w, 8, seed=n_shots), TOL[w.dtype])
