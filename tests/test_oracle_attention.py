"""Pins of the oracle's key sets, forward attention and backward (CPU only).

Each check compares the oracle with something other than itself: a dense full-matrix softmax,
torch's scaled_dot_product_attention with an explicit boolean mask (a library routine, forward
and autograd backward), masks derived in the test from the layout rules stated on the pages,
constant-V and finite-difference identities."""
import math

import numpy as np
import pytest
import torch

import moc_inputs as mi
from oracle import moc_oracle as mo

torch.set_default_dtype(torch.float64)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _mask_from_rules(layout, sel):
    """M[b,h,t,j] = key j is visible to query t, derived directly from the page rules:
    every text key; every key whose chunk has the query's shot id (text queries: the text);
    every key of a routed chunk."""
    off = np.asarray(layout.chunk_offsets)
    shot = np.asarray(layout.chunk_shot)
    L = int(off[-1])
    tok_chunk = np.zeros(L, dtype=np.int64)
    for c in range(len(shot)):
        tok_chunk[off[c]:off[c + 1]] = c
    tok_shot = shot[tok_chunk]
    B, H, _, S = sel.shape
    M = np.zeros((B, H, L, L), dtype=bool)
    is_text_key = np.zeros(L, dtype=bool)
    is_text_key[layout.text_begin:layout.text_end] = True
    for b in range(B):
        for h in range(H):
            for t in range(L):
                row = is_text_key | (tok_shot == tok_shot[t])
                for c in sel[b, h, t]:
                    if c >= 0:
                        row[off[c]:off[c + 1]] = True
                M[b, h, t] = row
    return M


def _sdpa(Q, K, V, M, scale):
    q = torch.tensor(Q, requires_grad=True)
    k = torch.tensor(K, requires_grad=True)
    v = torch.tensor(V, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=torch.tensor(M),
                                                         scale=scale)
    s = (q @ k.transpose(-1, -2)) * scale
    s = s.masked_fill(~torch.tensor(M), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return q, k, v, o, lse


def _route_random(layout, B, H, d, top_k, causal, seed):
    Q = _rand((B, H, layout.L, d), seed)
    K = _rand((B, H, layout.L, d), seed + 1)
    kb = mo.pool_keys(K, layout)
    r = mo.route(Q, kb, layout, top_k, causal)
    return Q, K, r


def test_dense_equivalence_tiny_layout():
    """top_k = all chunks, no causal mask -> MoC equals dense softmax(QK^T/sqrt(d))V
    (Mixture of Contexts summary §3.1: dense attention definition)."""
    w = mi.tiny()
    lay = w.layout
    # tiny layout, reduced head shape to keep the CPU suite short
    B, H, d = 1, 1, 16
    Q, K, r = _route_random(lay, B, H, d, top_k=lay.C, causal=False, seed=11)
    V = _rand((B, H, lay.L, d), 13)
    O, lse = mo.attend(Q, K, V, lay, r.sel)
    s = (Q[0, 0] @ K[0, 0].T) / math.sqrt(d)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    Od = (p / p.sum(axis=1, keepdims=True)) @ V[0, 0]
    lsed = (m[:, 0] + np.log(p.sum(axis=1)))
    assert np.max(np.abs(O[0, 0] - Od)) < 1e-12
    assert np.max(np.abs(lse[0, 0] - lsed)) < 1e-10
    pairs = mo.pair_counts(lay, r.sel)
    assert int(pairs[0, 0]) == lay.L * lay.L


@pytest.mark.parametrize("seed", range(6))
def test_masked_sdpa_equivalence_random_layouts(seed):
    """Any routing: oracle forward, LSE and backward equal torch SDPA (fp64, CPU) with the
    mask M[t,j] = [j in Omega(t)] built from the page rules."""
    rng = np.random.default_rng(100 + seed)
    lay = mi.make_random_layout(rng, max_shots=4, max_frames=3, max_chunk=12)
    B, H, d = 2, 2, 8
    top_k = int(rng.integers(0, lay.C + 1))
    causal = bool(seed % 2)
    Q, K, r = _route_random(lay, B, H, d, top_k, causal, seed=200 + seed)
    V = _rand((B, H, lay.L, d), 300 + seed)
    dO = _rand((B, H, lay.L, d), 400 + seed)
    scale = 0.37
    O, lse = mo.attend(Q, K, V, lay, r.sel, scale=scale)
    M = _mask_from_rules(lay, r.sel)
    q, k, v, o, lse_t = _sdpa(Q, K, V, M, scale)
    assert np.max(np.abs(O - o.detach().numpy())) < 1e-12
    assert np.max(np.abs(lse - lse_t.detach().numpy())) < 1e-12
    (o * torch.tensor(dO)).sum().backward()
    dQ, dK, dV = mo.attend_bwd(Q, K, V, dO, lay, r.sel, scale=scale)
    assert np.max(np.abs(dQ - q.grad.numpy())) < 1e-11
    assert np.max(np.abs(dK - k.grad.numpy())) < 1e-11
    assert np.max(np.abs(dV - v.grad.numpy())) < 1e-11
    # dQ of single rows (what the full-size GPU test samples) against the same SDPA gradient
    rows = [(b, h, int(t)) for b in range(B) for h in range(H)
            for t in rng.choice(lay.L, size=min(5, lay.L), replace=False)]
    dq_rows = mo.attend_bwd_dq_rows(Q, K, V, dO, lay, r.sel, rows, scale=scale)
    want = np.stack([q.grad.numpy()[row] for row in rows])
    assert np.max(np.abs(dq_rows - want)) < 1e-11
    # the same rows from bf16 torch tensors (the GPU tests' inputs) equal the rows computed from
    # the bf16 values in fp64
    tb = [torch.tensor(x).to(torch.bfloat16) for x in (Q, K, V, dO)]
    fb = [x.double().numpy() for x in tb]
    a = mo.attend_bwd_dq_rows(*tb, lay, r.sel, rows, scale=scale)
    b = mo.attend_bwd_dq_rows(*fb, lay, r.sel, rows, scale=scale)
    assert np.array_equal(a, b)
    # every softmax row sums to one and every dS row to zero, so over all keys
    # sum_j dV_j = sum_t dO_t and sum_j dK_j = 0 (per b, h and dimension)
    assert np.max(np.abs(dV.sum(axis=2) - dO.sum(axis=2))) < 1e-11
    assert np.max(np.abs(dK.sum(axis=2))) < 1e-11
    # both sides are scale * sum over pairs of dS_tj (q_t . k_j): sum_t q_t.dQ_t = sum_j k_j.dK_j
    lhs = np.einsum("bhtd,bhtd->bh", Q, dQ)
    rhs = np.einsum("bhtd,bhtd->bh", K, dK)
    assert np.max(np.abs(lhs - rhs)) < 1e-11
    # anchors are always inside Omega (the text tokens and the own shot are mandatory)
    D = mo.derive(lay)
    for t in range(lay.L):
        ks = set(mo.key_set(D, t, r.sel[0, 0, t]).tolist())
        assert set(mo.anchor_keys(D, t).tolist()) <= ks


def test_causal_all_is_shot_block_causal():
    """top_k = all with the causal routing mask: a frame query sees the text, its own shot and
    every earlier shot (text first); a text query sees only the text (summary §3.2)."""
    lay = mi.build_layout(5, [2, 1, 3], 4)
    B, H, d = 1, 1, 8
    Q, K, r = _route_random(lay, B, H, d, top_k=lay.C, causal=True, seed=5)
    D = mo.derive(lay)
    shot_start = {}
    for c in range(lay.C):
        s = int(lay.chunk_shot[c])
        if s >= 0 and s not in shot_start:
            shot_start[s] = int(lay.chunk_offsets[c])
    for t in range(lay.L):
        keys = set(mo.key_set(D, t, r.sel[0, 0, t]).tolist())
        s = int(lay.chunk_shot[D.chunk_of[t]])
        if s < 0:
            expect = set(range(lay.text_begin, lay.text_end))
        else:
            end_own = max(int(lay.chunk_offsets[c + 1]) for c in range(lay.C)
                          if int(lay.chunk_shot[c]) == s)
            expect = set(range(0, end_own))
        assert keys == expect, t


def test_topk_zero_is_text_plus_own_shot():
    lay = mi.build_layout(3, [2, 2], 5)
    Q, K, r = _route_random(lay, 1, 1, 4, top_k=0, causal=True, seed=9)
    assert r.sel.shape[-1] == 0
    D = mo.derive(lay)
    for t in range(lay.L):
        s = int(lay.chunk_shot[D.chunk_of[t]])
        own = {j for j in range(lay.L) if int(lay.chunk_shot[D.chunk_of[j]]) == s}
        expect = own | set(range(lay.text_begin, lay.text_end))
        assert set(mo.key_set(D, t, []).tolist()) == expect


def test_constant_v_rows_give_that_row():
    lay = mi.build_layout(4, [3, 2], 6)
    Q, K, r = _route_random(lay, 1, 2, 8, top_k=2, causal=True, seed=21)
    row = _rand((8,), 22)
    V = np.broadcast_to(row, (1, 2, lay.L, 8)).copy()
    O, _ = mo.attend(Q, K, V, lay, r.sel)
    assert np.max(np.abs(O - row)) < 1e-13


def test_backward_finite_differences():
    """Central differences of f = sum(O * dO) with the routing frozen."""
    lay = mi.build_layout(3, [2, 2], 4)
    B, H, d = 1, 1, 4
    Q, K, r = _route_random(lay, B, H, d, top_k=1, causal=True, seed=31)
    V = _rand((B, H, lay.L, d), 32)
    dO = _rand((B, H, lay.L, d), 33)
    scale = 1.0 / math.sqrt(d)
    dQ, dK, dV = mo.attend_bwd(Q, K, V, dO, lay, r.sel, scale)

    def f(Q_, K_, V_):
        O, _ = mo.attend(Q_, K_, V_, lay, r.sel, scale)
        return float(np.sum(O * dO))

    eps = 1e-6
    for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        num = np.zeros_like(X)
        it = np.nditer(X, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            Xp = X.copy(); Xp[idx] += eps
            Xm = X.copy(); Xm[idx] -= eps
            args = {"Q": (Q, K, V), "K": (Q, K, V), "V": (Q, K, V)}[name]
            if name == "Q":
                fp, fm = f(Xp, K, V), f(Xm, K, V)
            elif name == "K":
                fp, fm = f(Q, Xp, V), f(Q, Xm, V)
            else:
                fp, fm = f(Q, K, Xp), f(Q, K, Xm)
            num[idx] = (fp - fm) / (2 * eps)
        err = np.max(np.abs(num - G)) / max(1e-12, np.max(np.abs(G)))
        assert err < 1e-7, (name, err)


@pytest.mark.parametrize("seed", range(4))
def test_attend_heads_equals_masked_sdpa(seed):
    """attend_heads (every row of a head, queries grouped by anchor set, row blocks of 3 so that
    groups split) against torch SDPA with the rule-built mask, forward, LSE and autograd
    backward, on random layouts with drop-off / drop-in noise (routed sets of varying size)."""
    rng = np.random.default_rng(700 + seed)
    lay = mi.make_random_layout(rng, max_shots=4, max_frames=3, max_chunk=11,
                                frame_is_shot=seed == 3)
    B, H, d = 2, 2, 8
    top_k = int(rng.integers(0, lay.C + 1))
    causal = seed % 2 == 0
    Q, K, r = _route_random(lay, B, H, d, top_k, causal, seed=800 + seed)
    sel, _ = mo.drop_noise(r, lay, causal, 0.5, 1.5, 4, seed)
    V = _rand((B, H, lay.L, d), 900 + seed)
    dO = _rand((B, H, lay.L, d), 950 + seed)
    scale = 0.29
    heads = [(b, h) for b in range(B) for h in range(H)]
    O, lse, dQ, dK, dV = mo.attend_heads(Q, K, V, lay, sel, heads, scale=scale, dO=dO, block=3)
    M = _mask_from_rules(lay, sel)
    q, k, v, o, lse_t = _sdpa(Q, K, V, M, scale)
    (o * torch.tensor(dO)).sum().backward()
    for (b, h) in heads:
        assert np.max(np.abs(O[(b, h)] - o.detach().numpy()[b, h])) < 1e-12
        assert np.max(np.abs(lse[(b, h)] - lse_t.detach().numpy()[b, h])) < 1e-12
        assert np.max(np.abs(dQ[(b, h)] - q.grad.numpy()[b, h])) < 1e-11
        assert np.max(np.abs(dK[(b, h)] - k.grad.numpy()[b, h])) < 1e-11
        assert np.max(np.abs(dV[(b, h)] - v.grad.numpy()[b, h])) < 1e-11
    # forward only returns the same O and LSE
    O2, lse2 = mo.attend_heads(Q, K, V, lay, sel, heads[:1], scale=scale)
    assert np.max(np.abs(O2[heads[0]] - O[heads[0]])) < 1e-13


def test_attend_heads_rejects_routed_sets_overlapping_the_anchors():
    lay = mi.build_layout(3, [2, 2], 4)
    Q, K, r = _route_random(lay, 1, 1, 4, top_k=1, causal=True, seed=41)
    V = _rand((1, 1, lay.L, 4), 42)
    bad = r.sel.copy()
    t = lay.L - 1
    bad[0, 0, t, 0] = int(mo.derive(lay).chunk_of[t])  # its own chunk (own shot)
    with pytest.raises(ValueError):
        mo.attend_heads(Q, K, V, lay, bad, [(0, 0)])
    bad = np.concatenate([r.sel, r.sel], axis=-1)  # every routed chunk listed twice
    with pytest.raises(ValueError):
        mo.attend_heads(Q, K, V, lay, bad, [(0, 0)])
