"""Selection checks shared by the GPU parity tests (imported by them; collects no tests).

The bar for chunk selections: identical to the oracle's as sets, except for queries whose
oracle k-th vs (k+1)-th score gap is below 1e-4 of the larger magnitude (route()'s tie report).
Those exempt queries are still checked:
  * the GPU's set is legal for the query (every chunk a candidate by the oracle's predicate,
    ascending, unique, -1 padded) and of the oracle's size;
  * noise-free, it differs from the oracle's only inside the near-tie band: every chunk the GPU
    picked scores (fp64, from the same inputs) at least the oracle's k-th score less 1e-4 of
    the larger magnitude;
and the exemption itself is bounded: the oracle flags few queries (a flag set too broadly would
empty the check), and few of the flagged queries differ.
"""
import numpy as np

from oracle import moc_oracle as mo

# oracle-flagged queries: measured 0 .. 1.1e-3 on the parity workloads (single-shot 64-token chunks
# the most); denser candidate sets flag more (8e-3 with 1,023 candidates and top-32)
TIE_FRAC_MAX = 5e-3
DIFF_FRAC_MAX = 1e-4       # flagged queries whose GPU set differs, per checked query
DIFF_ABS_MIN = 8           # ... but at least this many are allowed on small inputs


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def allowed_table(D, causal, cand_mask_bh=None):
    """bool [C, C]: chunk c is a routing candidate of a query in chunk cq (the oracle's
    predicate), and set in the outer-routing mask row when one is given."""
    A = np.array([[mo.allowed(D, cq, c, causal) for c in range(D.C)] for cq in range(D.C)])
    if cand_mask_bh is not None:
        A &= cand_mask_bh
    return A


def check_legal(layout, sel, nsel, top_k, causal, exact_count=True, cand_mask=None,
                heads=None, A0=None):
    """Every row of the listed heads (all by default), vectorised: listed chunks are candidates,
    ascending and unique, the rest of the row is -1, and (exact_count) there are
    min(k, #candidates) of them."""
    D = mo.derive(layout)
    B, H, L, S = sel.shape
    cq = D.chunk_of
    if A0 is None and cand_mask is None:
        A0 = allowed_table(D, causal)
    for (b, h) in (heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]):
        A = A0 if cand_mask is None else allowed_table(D, causal, cand_mask[b, h])
        s = sel[b, h].astype(np.int64)
        n = nsel[b, h].astype(np.int64)
        assert np.all((n >= 0) & (n <= S)), (b, h)
        valid = np.arange(S)[None, :] < n[:, None]
        assert np.all(s[~valid] == -1), (b, h, "padding")
        assert np.all(s[valid] >= 0) and np.all(s[valid] < D.C), (b, h, "range")
        ok = A[np.repeat(cq, S).reshape(L, S)[valid], s[valid]]
        bad = np.nonzero(~ok)[0]
        assert ok.all(), (b, h, "not a candidate", int(bad.size))
        if S > 1:
            inc = s[:, 1:] > s[:, :-1]
            assert np.all(inc | ~valid[:, 1:]), (b, h, "not ascending/unique")
        if exact_count:
            need = np.minimum(min(int(top_k), D.C), A.sum(axis=1))[cq]
            assert np.array_equal(n, need), (b, h, "count")


def check_selection(layout, gsel, gnsel, o_sel, o_nsel, o_route, Q, kbar, causal, noise=False,
                    rows=None, label="", tie_frac_max=TIE_FRAC_MAX):
    """GPU selections (gsel, gnsel) against the oracle's (o_sel, o_nsel; o_route is the
    oracle's noise-free routing with its tie report). rows = list of (b, h, t) to check, or None
    for every row. Returns the number of flagged queries whose set differs."""
    exempt = o_route.gap_exempt
    k_eff = o_route.k_eff
    if rows is None:
        g = np.sort(gsel[..., :o_sel.shape[-1]] if gsel.shape[-1] >= o_sel.shape[-1] else gsel, -1)
        same = np.all(g == np.sort(o_sel, -1), -1) & (gnsel == o_nsel)
        if gsel.shape[-1] > o_sel.shape[-1]:
            same &= np.all(gsel[..., o_sel.shape[-1]:] == -1, -1)
        diff = np.argwhere(~same)
        n_rows = same.size
        tie_frac = float(exempt.mean())
    else:
        diff = []
        for (b, h, t) in rows:
            a = sorted(int(c) for c in gsel[b, h, t] if c >= 0)
            o = sorted(int(c) for c in o_sel[b, h, t] if c >= 0)
            if a != o or int(gnsel[b, h, t]) != int(o_nsel[b, h, t]):
                diff.append((b, h, t))
        diff = np.asarray(diff, dtype=np.int64).reshape(-1, 3)
        n_rows = len(rows)
        tie_frac = float(np.mean([exempt[r] for r in rows]))
    not_exempt = [tuple(r) for r in diff if not exempt[tuple(r)]]
    assert not not_exempt, f"{label}: {len(not_exempt)} selections differ, first {not_exempt[:5]}"
    say(f"{label}: {n_rows} rows, oracle near-ties {tie_frac:.2e}, "
        f"{len(diff)} flagged rows differ")
    assert tie_frac < tie_frac_max, (label, tie_frac)
    assert len(diff) <= max(DIFF_ABS_MIN, DIFF_FRAC_MAX * n_rows), (label, len(diff), n_rows)
    D = mo.derive(layout)
    for (b, h, t) in (tuple(int(x) for x in r) for r in diff):
        cq = int(D.chunk_of[t])
        cand = set(int(c) for c in mo.candidates(D, cq, causal))
        g = [int(c) for c in gsel[b, h, t, :gnsel[b, h, t]]]
        assert all(c in cand for c in g) and g == sorted(set(g)), (label, b, h, t, g)
        assert all(int(c) == -1 for c in gsel[b, h, t, gnsel[b, h, t]:]), (label, b, h, t)
        if noise:
            continue
        assert len(g) == min(k_eff, len(cand)), (label, b, h, t, g)
        q = mo._as_f64(Q[b, h, t])
        kb = np.asarray(kbar[b, h], dtype=np.float64)
        o = [int(c) for c in o_sel[b, h, t, :o_nsel[b, h, t]]]
        sk = min(float(q @ kb[c]) for c in o)  # the oracle's k-th best score
        for c in g:
            sc = float(q @ kb[c])
            assert sc >= sk - mo.TIE_REL * max(abs(sk), abs(sc)), (label, b, h, t, c, sc, sk)
    return len(diff)
