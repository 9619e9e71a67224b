"""GPU parity of the training path: drop-off / drop-in routing noise (bit-exact generator words,
set parity with the tie exemption) and the attention backward (dQ, dK, dV against the oracle's
fp64 backward over the same routed sets, max-abs 1e-2 for bf16)."""
import numpy as np
import pytest
import torch

import moc_inputs as mi
import parity_checks as pc
from oracle import moc_oracle as mo

pytestmark = pytest.mark.gpu

TOL = 1e-2


_say = pc.say


def _run(w: mi.Workload, backward: bool):
    import sparse_chunk_routed_amd as moc
    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    _say(f"workload {w.name} L={w.L} C={w.C} B={w.B} H={w.H} d={w.d} k={w.top_k} "
         f"p_max={w.p_max} lam={w.lam}")
    Q, K, V, dO = mi.make_qkv(w, with_dout=True)
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    cfg = moc.RouteCfg(w.top_k, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed)
    Qd, Kd, Vd, dOd = (x.to(dev) for x in (Q, K, V, dO))
    r = moc.forward(Qd, Kd, Vd, lay, cfg)
    out = {"Q": Q, "K": K, "V": V, "dO": dO, "sel": r.sel.cpu().numpy(),
           "nsel": r.nsel.cpu().numpy(), "O": r.O.float().cpu().numpy(),
           "pairs": r.varlen.pair_count.cpu().numpy()}
    if backward:
        dQ, dK, dV = moc.attend_bwd(Qd, Kd, Vd, r.O, r.lse, dOd, lay, r.varlen)
        torch.cuda.synchronize()
        out.update(dQ=dQ.float().cpu().numpy(), dK=dK.float().cpu().numpy(),
                   dV=dV.float().cpu().numpy())
    torch.cuda.synchronize()
    _say("gpu path done")
    return out


def _check_noise(w, g, tie_frac_max=pc.TIE_FRAC_MAX):
    """GPU selections vs oracle route + drop noise (parity_checks.check_selection: exempt
    near-tie queries only need legal sets); returns the number of rows the noise changed."""
    kb = mo.pool_keys(g["K"], w.layout)
    r = mo.route(g["Q"], kb, w.layout, w.top_k, w.causal)
    sel, nsel = mo.drop_noise(r, w.layout, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed)
    pc.check_selection(w.layout, g["sel"], g["nsel"], sel, nsel, r, g["Q"], kb, w.causal,
                       noise=w.p_max > 0 or w.lam > 0, label=f"{w.name} noise",
                       tie_frac_max=tie_frac_max)
    pc.check_legal(w.layout, g["sel"], g["nsel"], w.top_k, w.causal,
                   exact_count=not (w.p_max > 0 or w.lam > 0))
    # the causal DAG survives the noise (drop-in only draws causal candidates)
    if w.causal:
        assert mo.is_dag(w.C, mo.routed_edges(w.layout, g["sel"]))
    assert np.array_equal(g["pairs"], mo.pair_counts(w.layout, g["sel"]))
    return int((nsel != r.nsel).sum())


def _check_grads(w, g):
    dQ, dK, dV = mo.attend_bwd(g["Q"], g["K"], g["V"], g["dO"], w.layout, g["sel"])
    for name, a, b in (("dQ", g["dQ"], dQ), ("dK", g["dK"], dK), ("dV", g["dV"], dV)):
        err = float(np.max(np.abs(a - b)))
        rel = err / max(1e-30, float(np.max(np.abs(b))))
        _say(f"{name}: max|err|={err:.3e} (max|ref|={np.max(np.abs(b)):.3e}, rel {rel:.2e})")
        assert err <= TOL, (name, err)
        assert rel <= 2e-2, (name, rel)


@pytest.mark.parametrize("k", [2, 4])
def test_noise_and_backward_slice(k):
    """The 4,224-token gradient slice at the headline head shape; k=4 so drop-off fires."""
    w = mi.grad_slice(top_k=k)
    g = _run(w, backward=True)
    changed = _check_noise(w, g)
    assert changed > 0  # drop-in (lambda=1) changes many selections
    _check_grads(w, g)


@pytest.mark.parametrize("seed", range(6))
def test_backward_random_layouts(seed):
    rng = np.random.default_rng(500 + seed)
    lay = mi.make_random_layout(rng, max_shots=4, max_frames=3, max_chunk=200,
                                frame_is_shot=seed in (2, 5))
    w = mi.Workload(f"bwd{seed}", 2, 2, [64, 128, 64, 128, 64, 128][seed], "bf16", lay,
                    top_k=min(lay.C, [1, 3, 2, 0, 4, 2][seed]), causal=seed not in (1, 4),
                    clustered_keys=True, p_max=[0.0, 0.5, 0.3, 0.2, 0.0, 0.4][seed],
                    lam=[0.0, 2.0, 1.0, 0.5, 1.5, 0.0][seed], seed=seed)
    g = _run(w, backward=True)
    _check_noise(w, g)
    _check_grads(w, g)


def test_noise_headline_sampled():
    """Training-noise routing at the headline size (the train workload): 400 sampled queries
    of every head against the oracle's route plus noise."""
    w = mi.train()
    g = _run(w, backward=False)
    kb = mo.pool_keys(g["K"], w.layout)
    r = mo.route(g["Q"], kb, w.layout, w.top_k, w.causal)
    rng = np.random.default_rng(0)
    rows = [(0, h, int(t)) for h in range(w.H) for t in rng.choice(w.L, 400, replace=False)]
    sel, nsel = mo.drop_noise(r, w.layout, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed,
                              rows=rows)
    pc.check_selection(w.layout, g["sel"], g["nsel"], sel, nsel, r, g["Q"], kb, w.causal,
                       noise=True, rows=rows, label="train sampled")
    pc.check_legal(w.layout, g["sel"], g["nsel"], w.top_k, w.causal, exact_count=False)
    assert np.array_equal(g["pairs"], mo.pair_counts(w.layout, g["sel"]))


def _check_full_heads(w, g, heads, tol=TOL):
    """dQ, dK, dV (and the forward O) of every row of the listed heads against the oracle's
    fp64 attention over the same key sets (attend_heads). The selections of these heads were
    checked against the oracle's before (every differing row a legal near-tie)."""
    O, lse, dQ, dK, dV = mo.attend_heads(g["Q"], g["K"], g["V"], w.layout, g["sel"], heads,
                                         dO=g["dO"])
    for (b, h) in heads:
        err = float(np.max(np.abs(g["O"][b, h] - O[(b, h)])))
        _say(f"head {h}: O max|err|={err:.3e}")
        assert err <= tol, err
        for name, a, ref in (("dQ", g["dQ"][b, h], dQ[(b, h)]), ("dK", g["dK"][b, h], dK[(b, h)]),
                             ("dV", g["dV"][b, h], dV[(b, h)])):
            e = np.abs(a - ref)
            err = float(e.max())
            rel = err / max(1e-30, float(np.max(np.abs(ref))))
            worst = np.unravel_index(int(np.argmax(e)), e.shape)
            _say(f"head {h} {name}: max|err|={err:.3e} at {worst} "
                 f"(max|ref|={np.max(np.abs(ref)):.3e}, rel {rel:.2e})")
            assert err <= tol, (h, name, err)
            assert rel <= 2e-2, (h, name, rel)


def test_backward_short_noise_full_heads():
    """The short 33,016-token layout (256 text + 21 frames, frame = shot) with the training
    noise of the train workload (p_max 0.3, lambda 1): 12 heads on the GPU; every selection
    checked, and O, dQ, dK, dV of two whole heads against the oracle. Text keys are split into
    three query ranges here, whose partial gradients are summed in order."""
    w = mi.short(p_max=0.3, lam=1.0, max_drop_in=8)
    g = _run(w, backward=True)
    changed = _check_noise(w, g)
    assert changed > 0
    _check_full_heads(w, g, [(0, 0), (0, 11)])


def test_backward_train_full_head():
    """The backward at full size: the train workload (175,232 tokens, 12 heads, routing noise)
    that the train benchmark times.
    * Head 0: every selection against the oracle's route plus noise, then O, dQ, dK and dV of
      every row and key against the oracle's fp64 attention (the text keys' 11 query splits,
      the gathered bucket images, key tiles late in the sequence).
    * Every head: dQ on sampled rows, and over every key sum_j dV_j = sum_t dO_t: each query's
      softmax sums to one. The kernel rounds P to bf16 before the dV MFMAs, so a query's P sums
      to one within 2^-9 at worst. Against standard-normal dO the error of sum_t eps_t dO_t has
      a standard deviation of at most 2^-9 sqrt(L); the tolerance is 4 of those, 2^-7 sqrt(L)
      (about 3.3 against a signal of about sqrt(L) = 418)."""
    w = mi.train()
    g = _run(w, backward=True)
    # head 0 alone: the generator counter of (b, h) = (0, 0) does not depend on H
    kb = mo.pool_keys(g["K"][:, :1], w.layout)
    r = mo.route(g["Q"][:, :1], kb, w.layout, w.top_k, w.causal)
    sel, nsel = mo.drop_noise(r, w.layout, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed)
    pc.check_selection(w.layout, g["sel"][:, :1], g["nsel"][:, :1], sel, nsel, r,
                       g["Q"][:, :1], kb, w.causal, noise=True, label="train head 0")
    pc.check_legal(w.layout, g["sel"], g["nsel"], w.top_k, w.causal, exact_count=False)
    _check_full_heads(w, g, [(0, 0)])
    # sampled dQ rows of every other head, over the oracle's own routing plus noise
    kb_all = mo.pool_keys(g["K"], w.layout)
    r_all = mo.route(g["Q"], kb_all, w.layout, w.top_k, w.causal)
    rng = np.random.default_rng(7)
    rows = [(0, h, int(t)) for h in range(1, w.H) for t in rng.choice(w.L, 6, replace=False)]
    osel, onsel = mo.drop_noise(r_all, w.layout, w.causal, w.p_max, w.lam, w.max_drop_in,
                                w.seed, rows=rows)
    pc.check_selection(w.layout, g["sel"], g["nsel"], osel, onsel, r_all, g["Q"], kb_all,
                       w.causal, noise=True, rows=rows, label="train dQ rows")
    ref = mo.attend_bwd_dq_rows(g["Q"], g["K"], g["V"], g["dO"], w.layout, g["sel"], rows)
    got = np.stack([g["dQ"][row] for row in rows])
    err = float(np.max(np.abs(got - ref)))
    _say(f"dQ rows={len(rows)}: max|err|={err:.3e} (max|ref|={np.max(np.abs(ref)):.3e})")
    assert err <= TOL, err
    dv_sum = g["dV"].astype(np.float64).sum(axis=2)
    do_sum = g["dO"].double().sum(dim=2).numpy()
    derr = float(np.max(np.abs(dv_sum - do_sum)))
    tol = 2.0 ** -7 * np.sqrt(w.L)
    _say(f"sum_j dV_j vs sum_t dO_t: max|diff|={derr:.3e} (tol {tol:.2f}, "
         f"max|sum dO|={np.max(np.abs(do_sum)):.1f})")
    assert derr <= tol, derr
