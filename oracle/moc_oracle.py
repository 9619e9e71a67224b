"""Plain CPU oracle of the Mixture-of-Contexts (MoC) attention layer, in IEEE binary64.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
may import or call this module. It shares no code with the HIP path (sparse_chunk_routed_amd)
and imports nothing from it; the only common module is moc_inputs (seeded inputs, no method
arithmetic).

Sources (page titles; section / equation named, no line numbers):
  [MoC-S]  "Mixture of Contexts for Long Video Generation | Summary" (greeksharifa.github.io):
           §3.1 Mixture of Contexts, §3.2 Attention Chunking and Routing, §3.3 Computation
           Efficiency (Eq. 4, Eq. 5), Appendix A and G.
  [MoC-W]  jxzklqfsx.com write-up of the MoC paper: sections 上下文混合, 注意力塊劃分與路由
           (固定的跨模態選擇, 固定的鏡頭內選擇, 稀疏 MoC 中的因果性), 計算效率.
  [MoC-D]  docswell reading-group slides "Mixture of Contexts for Long Video Generation":
           slides 11 (Router), 12 (Causal Routing), 13 (Router constraints), 14 (drop-off/in).

What is computed (per batch element b and head h; routing is independent per head, [MoC-S] §3.1):
  1. Layout: chunks are contiguous token ranges aligned to the caption (text), frames and shots
     ([MoC-S] §3.2; [MoC-W] 內容對齊的塊劃分). Text chunks form one pseudo-shot.
  2. Pool: kbar_c = mean of the keys of chunk c ([MoC-D] slide 11; [MoC-S] §3.1). Reading: exact
     sum, one binary64 division by n_c, round-to-nearest-even to binary32.
  3. Candidates: chunk c is an optional candidate for query t iff c is not text, c is not in the
     query's own shot, and (if causal) c < chunk(t). Mandatory links are removed before top-k
     ([MoC-W] 計算效率: the pre-routing mask); causal masks edges i->j with j >= i ([MoC-S] §3.2).
  4. Score: s_c = q_t . kbar_c, a plain dot product, no router weights ([MoC-S] §3.1).
  5. Top-k: the min(k, #candidates) best candidates; an exact tie goes to the lower chunk index.
  6. Drop-off / drop-in (training noise, [MoC-S] §3.1; [MoC-D] slide 14): see drop_noise().
  7. Key set: Omega(t) = text tokens U own-shot tokens U tokens of the routed chunks
     ([MoC-S] §3.1-3.2; [MoC-W] 固定的跨模態選擇 / 固定的鏡頭內選擇).
  8. Attend: o_t = softmax(q_t K_Omega^T * scale) V_Omega, scale = 1/sqrt(d) by default
     ([MoC-S] §3.1); lse_t = natural log of the softmax denominator (with the max added back).
  9. Backward with Omega fixed (top-k is non-differentiable, [MoC-S] §3.1 and Appendix A).
 10. Counts: pairs = sum_t |Omega(t)|; FLOPs at 4*d per attended pair ([MoC-S] Eq. 5).
 11. Outer-loop context routing ([MoC-S] Appendix I): a coarse router picks, per query segment,
     the top-M segments by the dot product of mean-pooled features; inner routing (3-6) then
     only considers chunks of the query's own segment and of the picked segments. See
     route_outer().
 12. Quantised scores ([MoC-S] §5 Conclusion, [MoC-W] 結論, [MoC-D] slide 21 list quantisation
     among the directions for faster kernels, without fixing a format): Q and K in the OCP
     microscaling MXFP8 format (e4m3 elements, one power-of-two scale per 32 elements along d),
     attention (8) over the dequantised values. See mx_quantize().
 13. Quantised values (the same pages: quantisation and the key/value layout as directions):
     V in MXFP8 with its blocks of 32 along the key axis (per head and dim), attention (8) over
     dequantised Q, K and V (attend_mxv), and the bound on what rounding the softmax weights to
     e4m3 can add (pv_fp8_bound). See mx_quantize_keys().
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

from . import rng as _rng

TEXT_SHOT = -1  # pseudo-shot id of every text chunk


# ---------------------------------------------------------------------------------------------
# 1. Layout
# ---------------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Derived:
    L: int
    C: int
    offsets: np.ndarray        # int64 [C+1]
    sizes: np.ndarray          # int64 [C]
    shot: np.ndarray           # int64 [C]; TEXT_SHOT for text chunks
    is_text: np.ndarray        # bool [C]
    chunk_of: np.ndarray       # int64 [L]
    text_begin: int
    text_end: int


def derive(layout) -> Derived:
    """Validate a layout and derive per-token / per-chunk tables."""
    off = np.asarray(layout.chunk_offsets, dtype=np.int64)
    shot = np.asarray(layout.chunk_shot, dtype=np.int64)
    C = len(shot)
    if len(off) != C + 1 or off[0] != 0 or np.any(np.diff(off) <= 0):
        raise ValueError("chunk offsets must start at 0 and increase strictly")
    if np.any(shot < TEXT_SHOT):
        raise ValueError("shot ids are -1 (text) or >= 0")
    L = int(off[-1])
    tb, te = int(layout.text_begin), int(layout.text_end)
    is_text = np.zeros(C, dtype=bool)
    for c in range(C):
        a, b = int(off[c]), int(off[c + 1])
        inside = tb <= a and b <= te
        overlap = a < te and tb < b
        if overlap and not inside:
            raise ValueError("a chunk straddles the text range")
        is_text[c] = inside and tb < te
        if is_text[c] != (shot[c] == TEXT_SHOT):
            raise ValueError("text chunks must carry shot id -1, and only they")
    # each shot's chunks are contiguous
    seen = set()
    prev = None
    for c in range(C):
        s = int(shot[c])
        if s == TEXT_SHOT:
            prev = None
            continue
        if s != prev:
            if s in seen:
                raise ValueError("a shot's chunks must be contiguous")
            seen.add(s)
        prev = s
    if tb < te:
        # text chunks contiguous (one range)
        tidx = np.nonzero(is_text)[0]
        if int(off[tidx[0]]) != tb or int(off[tidx[-1] + 1]) != te:
            raise ValueError("text range must be a union of whole chunks")
    chunk_of = np.repeat(np.arange(C, dtype=np.int64), np.diff(off))
    return Derived(L, C, off, np.diff(off), shot, is_text, chunk_of, tb, te)


def shot_of_chunk(D: Derived, c: int) -> int:
    return int(D.shot[c])


def shot_range_tokens(D: Derived, s: int) -> np.ndarray:
    """All token indices whose chunk belongs to shot s (text tokens for the text pseudo-shot)."""
    cs = np.nonzero(D.shot == s)[0]
    return np.concatenate([np.arange(D.offsets[c], D.offsets[c + 1]) for c in cs])


def anchor_keys(D: Derived, t: int) -> np.ndarray:
    """Mandatory keys of query t: all text tokens and all tokens of the query's own shot.
    A text query's own shot is the text itself, so its anchor set is the text range."""
    s = int(D.shot[D.chunk_of[t]])
    own = shot_range_tokens(D, s)
    text = np.arange(D.text_begin, D.text_end)
    return np.union1d(text, own)


# ---------------------------------------------------------------------------------------------
# 2. Pool
# ---------------------------------------------------------------------------------------------

def pool_keys(K, layout) -> np.ndarray:
    """kbar[b,h,c,:] = RN32( RN64(exact sum of K over chunk c) / n_c ).  float32 [B,H,C,d]."""
    D = derive(layout)
    K = np.asarray(_as_f64(K))
    B, H, L, d = K.shape
    out = np.zeros((B, H, D.C, d), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for c in range(D.C):
                a, e = int(D.offsets[c]), int(D.offsets[c + 1])
                n = e - a
                cols = K[b, h, a:e, :].T.tolist()  # one list of n values per dimension
                for j in range(d):
                    s = math.fsum(cols[j])  # exact sum, rounded once to binary64
                    out[b, h, c, j] = np.float32(s / float(n))
    return out


# ---------------------------------------------------------------------------------------------
# 3-5. Candidates, scores, top-k
# ---------------------------------------------------------------------------------------------

def allowed(D: Derived, cq: int, c: int, causal: bool) -> bool:
    """Is chunk c an optional routing candidate for a query in chunk cq?"""
    if D.is_text[c]:
        return False
    if D.shot[c] == D.shot[cq]:
        return False
    if causal and not (c < cq):
        return False
    return True


def candidates(D: Derived, cq: int, causal: bool) -> np.ndarray:
    return np.array([c for c in range(D.C) if allowed(D, cq, c, causal)], dtype=np.int64)


@dataclass
class Routing:
    sel: np.ndarray     # int32 [B,H,L,S]: selected chunk ids ascending, -1 padded
    nsel: np.ndarray    # int32 [B,H,L]
    gap_exempt: np.ndarray  # bool [B,H,L]: k-th vs (k+1)-th score gap < 1e-4 relative
    k_eff: int


def scores(Q, kbar) -> np.ndarray:
    """s[b,h,t,c] = q_t . kbar_c in binary64 (bf16/fp32 inputs widen exactly)."""
    Q = _as_f64(Q)
    kb = np.asarray(kbar, dtype=np.float64)
    return np.einsum("bhtd,bhcd->bhtc", Q, kb, optimize=True)


TIE_REL = 1e-4


def route(Q, kbar, layout, top_k: int, causal: bool,
          cand_mask: Optional[np.ndarray] = None) -> Routing:
    """Top-min(k, #candidates) chunks per (b, h, t), stored ascending by chunk id. With
    cand_mask (bool [B,H,C,C], row = the query's chunk), a candidate must also be set in it.
    Scores are formed one head at a time (the same products as scores(), in less memory)."""
    D = derive(layout)
    B, H, L, _ = Q.shape
    C = D.C
    k_eff = min(int(top_k), C)
    sel = np.full((B, H, L, k_eff), -1, dtype=np.int32)
    nsel = np.zeros((B, H, L), dtype=np.int32)
    exempt = np.zeros((B, H, L), dtype=bool)
    cands = [candidates(D, cq, causal) for cq in range(C)]
    for b in range(B):
        for h in range(H):
            s_bh = scores(Q[b:b + 1, h:h + 1], np.asarray(kbar)[b:b + 1, h:h + 1])[0, 0]
            for cq in range(C):
                toks = np.arange(D.offsets[cq], D.offsets[cq + 1])
                cand = cands[cq] if cand_mask is None else cands[cq][cand_mask[b, h, cq, cands[cq]]]
                n = min(k_eff, len(cand))
                if n == 0:
                    continue
                sc = s_bh[np.ix_(toks, cand)]           # [nt, ncand]
                # order by (-score, chunk id): cand is ascending and the sort is stable
                order = np.argsort(-sc, axis=1, kind="stable")
                top = cand[order[:, :n]]
                sel[b, h, toks, :n] = np.sort(top, axis=1)
                nsel[b, h, toks] = n
                if len(cand) > n:
                    sk = np.take_along_axis(sc, order[:, n - 1:n], axis=1)[:, 0]
                    sk1 = np.take_along_axis(sc, order[:, n:n + 1], axis=1)[:, 0]
                    exempt[b, h, toks] = (sk - sk1) < TIE_REL * np.maximum(np.abs(sk), np.abs(sk1))
    return Routing(sel, nsel, exempt, k_eff)


# ---------------------------------------------------------------------------------------------
# 6. Context drop-off and drop-in
# ---------------------------------------------------------------------------------------------

def drop_noise_row(D: Derived, top: Sequence[int], b: int, h: int, t: int, H: int,
                   k_eff: int, causal: bool, p_max: float, lam: float, m_cap: int,
                   seed: int, thr: Optional[List[int]],
                   cand_row: Optional[np.ndarray] = None) -> List[int]:
    """Training-time routing noise for one query ([MoC-S] §3.1; [MoC-D] slide 14).

    Readings: drop-off removes min(floor(p*k), |T|) chunks from the routed top-k set T only
    (never the mandatory anchors), with p = u * p_max, u the top 24 bits of an H32 word;
    drop-in then adds min(m, |pool|) chunks from pool = candidates(t) minus T, with
    m ~ Poisson(lam) truncated at m_cap. Picks are uniform without replacement via
    idx = (H32 * remaining) >> 32 over the ascending list of what remains."""
    L = D.L
    T = sorted(int(c) for c in top)
    kept = list(T)
    if p_max > 0.0:
        r = _rng.h32(seed, _rng.counter(b, h, t, _rng.STREAM_DROP_P, 0, H, L))
        u = float(r >> 8) * (2.0 ** -24)
        p = u * float(np.float32(p_max))
        nd = min(int(math.floor(p * float(k_eff))), len(kept))
        for j in range(nd):
            w = _rng.h32(seed, _rng.counter(b, h, t, _rng.STREAM_DROP_PICK, j, H, L))
            idx = (w * (len(kept))) >> 32
            kept.pop(idx)
    added: List[int] = []
    if lam > 0.0:
        r = _rng.h32(seed, _rng.counter(b, h, t, _rng.STREAM_IN_COUNT, 0, H, L))
        m = _rng.poisson_from_word(r, thr, m_cap)
        cq = int(D.chunk_of[t])
        pool = [int(c) for c in candidates(D, cq, causal) if int(c) not in T
                and (cand_row is None or cand_row[int(c)])]
        for j in range(min(m, len(pool))):
            w = _rng.h32(seed, _rng.counter(b, h, t, _rng.STREAM_IN_PICK, j, H, L))
            idx = (w * len(pool)) >> 32
            added.append(pool.pop(idx))
    return sorted(kept + added)


def drop_noise(routing: Routing, layout, causal: bool, p_max: float, lam: float,
               m_cap: int, seed: int, rows: Optional[Iterable[Tuple[int, int, int]]] = None,
               cand_mask: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Apply drop-off then drop-in. Returns (sel [B,H,L,S], nsel [B,H,L]) with
    S = k_eff + (m_cap if lam > 0 else 0). With `rows`, only those (b,h,t) are computed and
    the other rows are left at -1 / 0."""
    D = derive(layout)
    B, H, L, _ = routing.sel.shape
    k_eff = routing.k_eff
    S = k_eff + (m_cap if lam > 0.0 else 0)
    thr = _rng.poisson_thresholds(float(np.float32(lam)), m_cap) if lam > 0.0 else None
    sel = np.full((B, H, L, S), -1, dtype=np.int32)
    nsel = np.zeros((B, H, L), dtype=np.int32)
    it = rows if rows is not None else ((b, h, t) for b in range(B) for h in range(H)
                                        for t in range(L))
    for (b, h, t) in it:
        n = int(routing.nsel[b, h, t])
        top = routing.sel[b, h, t, :n]
        row = None if cand_mask is None else cand_mask[b, h, int(D.chunk_of[t])]
        out = drop_noise_row(D, top, b, h, t, H, k_eff, causal, p_max, lam, m_cap, seed, thr,
                             row)
        sel[b, h, t, :len(out)] = out
        nsel[b, h, t] = len(out)
    return sel, nsel


# ---------------------------------------------------------------------------------------------
# 7-8. Key sets and attention
# ---------------------------------------------------------------------------------------------

def key_set(D: Derived, t: int, sel_row: Sequence[int]) -> np.ndarray:
    """Omega(t) as a sorted array of key indices (a set: no key counted twice)."""
    parts = [anchor_keys(D, t)]
    for c in sel_row:
        c = int(c)
        if c < 0:
            continue
        parts.append(np.arange(D.offsets[c], D.offsets[c + 1]))
    return np.unique(np.concatenate(parts))


def attend_row(q: np.ndarray, Kbh: np.ndarray, Vbh: np.ndarray, keys: np.ndarray,
               scale: float) -> Tuple[np.ndarray, float]:
    x = (Kbh[keys] @ q) * scale
    m = float(np.max(x))
    w = np.exp(x - m)
    z = float(np.sum(w))
    o = (w @ Vbh[keys]) / z
    return o, m + math.log(z)


def attend(Q, K, V, layout, sel, scale: Optional[float] = None,
           rows: Optional[Sequence[Tuple[int, int, int]]] = None):
    """Forward attention over Omega. Full: returns (O [B,H,L,d] fp64, lse [B,H,L] fp64).
    With `rows` (a list of (b,h,t)): returns (O [n,d], lse [n]) for those rows."""
    D = derive(layout)
    Q = _as_f64(Q)
    K = _as_f64(K)
    V = _as_f64(V)
    B, H, L, d = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    sel = np.asarray(sel)
    if rows is None:
        O = np.zeros((B, H, L, d))
        lse = np.zeros((B, H, L))
        for b in range(B):
            for h in range(H):
                for t in range(L):
                    keys = key_set(D, t, sel[b, h, t])
                    O[b, h, t], lse[b, h, t] = attend_row(Q[b, h, t], K[b, h], V[b, h], keys, scale)
        return O, lse
    rows = list(rows)
    O = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for i, (b, h, t) in enumerate(rows):
        keys = key_set(D, t, sel[b, h, t])
        O[i], lse[i] = attend_row(Q[b, h, t], K[b, h], V[b, h], keys, scale)
    return O, lse


# ---------------------------------------------------------------------------------------------
# 9. Backward with Omega fixed
# ---------------------------------------------------------------------------------------------

def attend_bwd(Q, K, V, dO, layout, sel, scale: Optional[float] = None):
    """Gradients of sum(O * dO) w.r.t. Q, K, V with the routed sets held fixed.

    Per query t with P = softmax(x), x_j = q_t.k_j*scale over j in Omega(t):
      dV_j += P_j dO_t;  dP_j = dO_t . v_j;  dS_j = P_j (dP_j - sum_i P_i dP_i);
      dQ_t = scale * sum_j dS_j k_j;  dK_j += scale * dS_j q_t."""
    D = derive(layout)
    Q = _as_f64(Q)
    K = _as_f64(K)
    V = _as_f64(V)
    dO = _as_f64(dO)
    B, H, L, d = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    sel = np.asarray(sel)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        for h in range(H):
            Kbh, Vbh = K[b, h], V[b, h]
            for t in range(L):
                keys = key_set(D, t, sel[b, h, t])
                p, ds = _bwd_row(Q[b, h, t], Kbh, Vbh, dO[b, h, t], keys, scale)
                dV[b, h, keys] += np.outer(p, dO[b, h, t])
                dQ[b, h, t] = scale * (ds @ Kbh[keys])
                dK[b, h, keys] += scale * np.outer(ds, Q[b, h, t])
    return dQ, dK, dV


def _bwd_row(q, Kbh, Vbh, g, keys, scale):
    """P and dS of one query over its key set (the steps of attend_bwd for one row)."""
    x = (Kbh[keys] @ q) * scale
    p = np.exp(x - np.max(x))
    p /= np.sum(p)
    dp = Vbh[keys] @ g
    ds = p * (dp - np.dot(p, dp))
    return p, ds


def attend_bwd_dq_rows(Q, K, V, dO, layout, sel, rows: Sequence[Tuple[int, int, int]],
                       scale: Optional[float] = None) -> np.ndarray:
    """dQ of attend_bwd for the listed (b, h, t) rows only ([n, d]): a query's gradient
    depends on its own key set alone, so sampled rows of a large input cost one row each."""
    D = derive(layout)
    d = Q.shape[-1]  # NumPy array or torch tensor (bf16 included)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    sel = np.asarray(sel)
    out = np.zeros((len(rows), d))
    heads = {}
    for i, (b, h, t) in enumerate(rows):
        if (b, h) not in heads:  # one fp64 copy of K and V per head
            heads = {(b, h): (_as_f64(K[b, h]), _as_f64(V[b, h]))}
        Kbh, Vbh = heads[(b, h)]
        keys = key_set(D, t, sel[b, h, t])
        _, ds = _bwd_row(_as_f64(Q[b, h, t]), Kbh, Vbh, _as_f64(dO[b, h, t]), keys, scale)
        out[i] = scale * (ds @ Kbh[keys])
    return out


def anchor_groups(D: Derived) -> List[Tuple[np.ndarray, np.ndarray]]:
    """(queries, anchor keys) for every group of queries that share their anchor set: the text
    queries (anchor = the text) and, for every shot, the shot's queries (anchor = text U shot)."""
    out = []
    for s in sorted(set(int(x) for x in D.shot)):
        toks = shot_range_tokens(D, s)
        out.append((toks, anchor_keys(D, int(toks[0]))))
    return out


def attend_heads(Q, K, V, layout, sel, heads: Sequence[Tuple[int, int]],
                 scale: Optional[float] = None, dO=None, block: int = 1024):
    """Every query row of the listed (b, h) heads, forward (and backward when dO is given):
    the quantities of attend() and attend_bwd() for those heads, in fp64, for inputs too large
    for the one-row-at-a-time form. Plain torch CPU ops in float64 (its matrix products and
    elementwise functions use every host core).

    Omega(t) is the disjoint union of Anch(t) and the routed chunks of t (step 8): routed chunks
    are never text or own-shot chunks, and each is listed once. The softmax over Omega(t) is
    therefore taken over the concatenation of the query's scores on those parts - its maximum and
    its sum of exponentials are the maximum and the sum over the parts. Queries that share their
    anchor set are handled together, up to `block` rows at a time, so that the anchor scores of a
    block are one matrix product; the routed scores of a chunk are one product over the block's
    queries that routed to it. Within a row nothing is reordered beyond the summation order of
    the products and sums.

    Returns (O, lse) - or (O, lse, dQ, dK, dV) with dO - as dicts of float64 NumPy arrays keyed
    by (b, h): O, dQ, dK, dV [L, d] and lse [L]."""
    import torch
    D = derive(layout)
    d = Q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    sel = np.asarray(sel)
    f64 = torch.float64

    def t64(x):
        return torch.from_numpy(np.ascontiguousarray(_as_f64(x)))

    res = {k: {} for k in ("O", "lse", "dQ", "dK", "dV")}
    for (b, h) in heads:
        Qh, Kh, Vh = t64(Q[b, h]), t64(K[b, h]), t64(V[b, h])
        G = None if dO is None else t64(dO[b, h])
        L = Qh.shape[0]
        O = torch.zeros((L, d), dtype=f64)
        lse = torch.zeros(L, dtype=f64)
        if G is not None:
            dQ = torch.zeros((L, d), dtype=f64)
            dK = torch.zeros((L, d), dtype=f64)
            dV = torch.zeros((L, d), dtype=f64)
        for toks, akeys in anchor_groups(D):
            ak = torch.from_numpy(akeys)
            Ka, Va = Kh[ak], Vh[ak]
            for i0 in range(0, len(toks), block):
                qb_np = toks[i0:i0 + block]
                # routed parts: chunk -> rows of the block that routed to it
                parts = {}
                for i, t in enumerate(qb_np):
                    row = [int(c) for c in sel[b, h, t] if c >= 0]
                    own = D.shot[D.chunk_of[t]]
                    if len(set(row)) != len(row) or any(D.is_text[c] or D.shot[c] == own
                                                        for c in row):
                        raise ValueError(f"routed set of query {t} is not disjoint from its "
                                         "anchors or lists a chunk twice")
                    for c in row:
                        parts.setdefault(c, []).append(i)
                parts = [(torch.tensor(ix), slice(int(D.offsets[c]), int(D.offsets[c + 1])))
                         for c, ix in sorted(parts.items())]
                qb = torch.from_numpy(qb_np)
                Qb = Qh[qb]
                xa = (Qb @ Ka.T) * scale
                xr = [(Qb[ix] @ Kh[ks].T) * scale for ix, ks in parts]
                m = xa.amax(dim=1)
                for (ix, _), x in zip(parts, xr):
                    m.scatter_reduce_(0, ix, x.amax(dim=1), reduce="amax")
                ea = torch.exp(xa - m[:, None])
                er = [torch.exp(x - m[ix, None]) for (ix, _), x in zip(parts, xr)]
                z = ea.sum(dim=1)
                for (ix, _), e in zip(parts, er):
                    z.index_add_(0, ix, e.sum(dim=1))
                pa = ea / z[:, None]
                pr = [e / z[ix, None] for (ix, _), e in zip(parts, er)]
                o = pa @ Va
                for (ix, ks), p in zip(parts, pr):
                    o.index_add_(0, ix, p @ Vh[ks])
                O[qb] = o
                lse[qb] = m + torch.log(z)
                if G is None:
                    continue
                gb = G[qb]
                dpa = gb @ Va.T
                dpr = [gb[ix] @ Vh[ks].T for ix, ks in parts]
                Dt = (pa * dpa).sum(dim=1)
                for (ix, _), p, dp in zip(parts, pr, dpr):
                    Dt.index_add_(0, ix, (p * dp).sum(dim=1))
                dsa = pa * (dpa - Dt[:, None])
                dsr = [p * (dp - Dt[ix, None]) for (ix, _), p, dp in zip(parts, pr, dpr)]
                dq = dsa @ Ka
                for (ix, ks), ds in zip(parts, dsr):
                    dq.index_add_(0, ix, ds @ Kh[ks])
                dQ[qb] = scale * dq
                dK.index_add_(0, ak, scale * (dsa.T @ Qb))
                dV.index_add_(0, ak, pa.T @ gb)
                for (ix, ks), p, ds in zip(parts, pr, dsr):
                    dK[ks] += scale * (ds.T @ Qb[ix])
                    dV[ks] += p.T @ gb[ix]
        res["O"][(b, h)], res["lse"][(b, h)] = O.numpy(), lse.numpy()
        if G is not None:
            res["dQ"][(b, h)] = dQ.numpy()
            res["dK"][(b, h)] = dK.numpy()
            res["dV"][(b, h)] = dV.numpy()
    if dO is None:
        return res["O"], res["lse"]
    return res["O"], res["lse"], res["dQ"], res["dK"], res["dV"]


# ---------------------------------------------------------------------------------------------
# 10. Counts and invariants
# ---------------------------------------------------------------------------------------------

def pair_counts(layout, sel) -> np.ndarray:
    """int64 [B,H]: sum over queries of |Omega(t)| = |Anch(t)| + sum of routed chunk sizes
    (routed chunks are never text or own-shot chunks, so the two parts are disjoint)."""
    D = derive(layout)
    sel = np.asarray(sel)
    B, H, L, _ = sel.shape
    anch = np.zeros(D.C, dtype=np.int64)
    for c in range(D.C):
        anch[c] = len(anchor_keys(D, int(D.offsets[c])))
    anchor_total = int(anch[D.chunk_of].sum())
    out = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            s = sel[b, h]
            out[b, h] = anchor_total + int(D.sizes[s[s >= 0]].sum())
    return out


def attention_flops(pairs: int, d: int) -> int:
    """Forward attention FLOPs at 4*d per attended (query, key) pair ([MoC-S] Eq. 5)."""
    return 4 * d * int(pairs)


def dense_flops(L: int, d: int) -> int:
    """FLOPs_dense = 4 L^2 d for one head ([MoC-S] Eq. 5)."""
    return 4 * L * L * d


def routed_edges(layout, sel) -> set:
    """Chunk interaction edges (chunk(t) -> c) for every routed selection."""
    D = derive(layout)
    sel = np.asarray(sel)
    E = set()
    B, H, L, S = sel.shape
    for b in range(B):
        for h in range(H):
            for t in range(L):
                for c in sel[b, h, t]:
                    if c >= 0:
                        E.add((int(D.chunk_of[t]), int(c)))
    return E


def is_dag(C: int, edges: Iterable[Tuple[int, int]]) -> bool:
    """Kahn's topological sort over chunk nodes."""
    out = {i: set() for i in range(C)}
    indeg = [0] * C
    for (a, b) in edges:
        if b not in out[a]:
            out[a].add(b)
            indeg[b] += 1
    stack = [i for i in range(C) if indeg[i] == 0]
    seen = 0
    while stack:
        n = stack.pop()
        seen += 1
        for m in out[n]:
            indeg[m] -= 1
            if indeg[m] == 0:
                stack.append(m)
    return seen == C


def check_routing(layout, sel, nsel, top_k: int, causal: bool, exact_count: bool = True,
                  cand_mask: Optional[np.ndarray] = None) -> None:
    """Raise AssertionError unless every selection is a legal candidate (and set in cand_mask,
    if given), ascending and unique, and (exact_count) there are exactly min(k, #candidates) of
    them."""
    D = derive(layout)
    sel = np.asarray(sel)
    B, H, L, S = sel.shape
    for cq in range(D.C):
        cand0 = set(int(c) for c in candidates(D, cq, causal))
        for t in range(int(D.offsets[cq]), int(D.offsets[cq + 1])):
            for b in range(B):
                for h in range(H):
                    cand = cand0 if cand_mask is None else {
                        c for c in cand0 if cand_mask[b, h, cq, c]}
                    need = min(int(top_k), D.C, len(cand))
                    n = int(nsel[b, h, t])
                    row = [int(c) for c in sel[b, h, t, :n]]
                    assert all(c in cand for c in row), (b, h, t, row)
                    assert row == sorted(set(row)), (b, h, t, row)
                    assert all(int(c) == -1 for c in sel[b, h, t, n:]), (b, h, t)
                    if exact_count:
                        assert n == need, (b, h, t, n, need)


# ---------------------------------------------------------------------------------------------
# 11. Outer-loop context routing ([MoC-S] Appendix I)
# ---------------------------------------------------------------------------------------------
# Readings. The pages add a first, coarse level of routing for long generation: whole segments
# are ranked by how well the averaged features of the current block of queries match the
# averaged features of each candidate segment, and the ordinary MoC router then only looks at
# chunks inside the best M of them (plus the mandatory context).
#  * Segments are given: contiguous groups of whole chunks (seg_chunk[nseg+1], chunk offsets),
#    each all text chunks or all video chunks. Text is mandatory context, never a candidate.
#  * The current query block of a query is its own segment. Its feature is the mean of the
#    segment's queries; a candidate segment's feature is the mean of its keys. Both are pooled
#    like chunk keys (exact sum, one binary64 division, RN to binary32).
#  * Candidates of query segment sq: video segments s != sq, and s < sq when causal (the
#    autoregressive reading: a segment is generated after the ones it retrieves from).
#    Score = dot product in binary64; top-min(M, #candidates); an exact tie goes to the lower
#    segment index; stored ascending.
#  * Inner routing of a query t considers only chunks of seg(t) and of the picked segments, on
#    top of the usual candidate rule (3); drop-in draws from that restricted pool. The
#    mandatory anchors (text, own shot) are unchanged.

@dataclass(frozen=True)
class Segments:
    nseg: int
    chunk_off: np.ndarray     # int64 [nseg+1]
    tok_off: np.ndarray       # int64 [nseg+1]
    is_text: np.ndarray       # bool [nseg]
    seg_of_chunk: np.ndarray  # int64 [C]


def derive_segments(layout, seg_chunk) -> Segments:
    D = derive(layout)
    so = np.asarray(seg_chunk, dtype=np.int64)
    nseg = len(so) - 1
    if nseg < 1 or so[0] != 0 or so[-1] != D.C or np.any(np.diff(so) <= 0):
        raise ValueError("segment chunk offsets must start at 0, increase strictly, end at C")
    is_text = np.zeros(nseg, dtype=bool)
    for sg in range(nseg):
        t = D.is_text[so[sg]:so[sg + 1]]
        if t.any() and not t.all():
            raise ValueError("a segment mixes text and video chunks")
        is_text[sg] = bool(t.all())
    seg_of_chunk = np.repeat(np.arange(nseg, dtype=np.int64), np.diff(so))
    return Segments(nseg, so, D.offsets[so], is_text, seg_of_chunk)


@dataclass(frozen=True)
class _Layout:
    chunk_offsets: np.ndarray
    chunk_shot: np.ndarray
    text_begin: int
    text_end: int


def segment_layout(layout, seg_chunk):
    """The layout whose chunks are the segments (text segments keep shot id -1)."""
    G = derive_segments(layout, seg_chunk)
    shot = np.where(G.is_text, TEXT_SHOT, np.arange(G.nseg))
    return _Layout(G.tok_off, shot, int(layout.text_begin), int(layout.text_end))


@dataclass
class OuterRouting:
    seg_sel: np.ndarray     # int32 [B,H,nseg,Msel]: picked segments ascending, -1 padded
    seg_nsel: np.ndarray    # int32 [B,H,nseg]
    gap_exempt: np.ndarray  # bool [B,H,nseg]: M-th vs (M+1)-th score gap < TIE_REL relative
    cand_mask: np.ndarray   # bool [B,H,C,C]: chunks the inner router may consider, per chunk
    qseg: np.ndarray        # float32 [B,H,nseg,d]
    kseg: np.ndarray        # float32 [B,H,nseg,d]


def segment_candidates(G: Segments, sq: int, causal: bool) -> List[int]:
    return [s for s in range(G.nseg)
            if not G.is_text[s] and s != sq and (not causal or s < sq)]


def route_outer(Q, K, layout, seg_chunk, M: int, causal: bool) -> OuterRouting:
    """Coarse top-M segment selection per (b, h, query segment) and the inner candidate mask."""
    G = derive_segments(layout, seg_chunk)
    D = derive(layout)
    slay = segment_layout(layout, seg_chunk)
    qseg = pool_keys(Q, slay)
    kseg = pool_keys(K, slay)
    B, H, nseg, d = qseg.shape
    msel = min(int(M), nseg)
    seg_sel = np.full((B, H, nseg, msel), -1, dtype=np.int32)
    seg_nsel = np.zeros((B, H, nseg), dtype=np.int32)
    exempt = np.zeros((B, H, nseg), dtype=bool)
    allowed_segs = np.zeros((B, H, nseg, nseg), dtype=bool)
    for b in range(B):
        for h in range(H):
            for sq in range(nseg):
                allowed_segs[b, h, sq, sq] = True
                cand = segment_candidates(G, sq, causal)
                n = min(msel, len(cand))
                if n == 0:
                    continue
                q = qseg[b, h, sq].astype(np.float64)
                sc = [float(np.dot(q, kseg[b, h, s].astype(np.float64))) for s in cand]
                order = sorted(range(len(cand)), key=lambda i: (-sc[i], cand[i]))
                top = sorted(cand[i] for i in order[:n])
                seg_sel[b, h, sq, :n] = top
                seg_nsel[b, h, sq] = n
                allowed_segs[b, h, sq, top] = True
                if len(cand) > n:
                    a, c = sc[order[n - 1]], sc[order[n]]
                    exempt[b, h, sq] = (a - c) < TIE_REL * max(abs(a), abs(c))
    cmask = allowed_segs[:, :, G.seg_of_chunk][:, :, :, G.seg_of_chunk]  # [B,H,C,C]
    return OuterRouting(seg_sel, seg_nsel, exempt, cmask, qseg, kseg)


# ---------------------------------------------------------------------------------------------
# 12. Quantised scores: MXFP8 Q and K
# ---------------------------------------------------------------------------------------------
# Readings. The pages name quantisation only as a direction for faster kernels ([MoC-S] §5;
# [MoC-W] 結論; [MoC-D] slide 21). This oracle fixes one published format and its plain
# conversion rule:
#  * Element format E4M3 of the OCP 8-bit floating point specification (OFP8): sign, 4 exponent
#    bits with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; the
#    all-ones exponent with mantissa 7 is NaN; no infinities; the largest finite value is 448.
#  * Shared scale of the OCP Microscaling (MX) specification v1.0: per block of 32 consecutive
#    elements of a row (along d), X = 2^E with E = floor(log2(max |x|)) - 8 (8 = the largest
#    exponent of E4M3), stored as the E8M0 code E + 127. Readings where the spec leaves a choice:
#    E is clamped below at -127 (the smallest E8M0 value), an all-zero block takes E = -127, and
#    the element x / X is rounded to the nearest E4M3 value with ties to the even code and
#    saturation at +-448 (|x / X| < 512, so only the top of the range clamps); the sign of a
#    value that rounds to zero is kept (code 0x80 for negative inputs).
#  * Attention then runs on the dequantised Q' = codes * X and K' = codes * X in exact
#    arithmetic (8); V stays in its input precision.

E4M3_MAX = 448.0
MX_BLOCK = 32
E4M3_EMAX = 8


def e4m3_value(code: int) -> float:
    """Value of an E4M3 code from its bit fields (NaN for the two NaN codes)."""
    code = int(code) & 0xFF
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return math.nan
    v = math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7)
    return -v if s else v


def e4m3_table() -> np.ndarray:
    """float64 [256]: the value of every code."""
    return np.array([e4m3_value(c) for c in range(256)])


def e4m3_round(v) -> np.ndarray:
    """Codes (uint8) of finite binary64 values: the nearest E4M3 value to min(|v|, 448), ties to
    the even code, sign from v (including a negative value that rounds to zero)."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("finite inputs only")
    mag = np.minimum(np.abs(v), E4M3_MAX)
    pos = e4m3_table()[:127]                       # codes 0..126, strictly increasing
    hi = np.clip(np.searchsorted(pos, mag, side="left"), 0, 126)   # first value >= mag
    lo = np.maximum(hi - 1, 0)
    dlo = mag - pos[lo]
    dhi = pos[hi] - mag
    take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(v)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def mx_scale_exponents(amax) -> np.ndarray:
    """E of blocks with largest magnitudes amax: floor(log2(amax)) - 8, at least -127; -127 for
    an all-zero block."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)  # amax = f 2^e with f in [0.5, 1): floor(log2 amax) = e - 1
    E = np.maximum(e.astype(np.int64) - 1 - E4M3_EMAX, -127)
    return np.where(amax == 0.0, -127, E)


def mx_quantize(X) -> Tuple[np.ndarray, np.ndarray]:
    """MXFP8 of X [..., d] (d a multiple of 32): codes uint8 [..., d] and E8M0 scale codes
    uint8 [..., d/32]."""
    X = _as_f64(X)
    d = X.shape[-1]
    if d % MX_BLOCK:
        raise ValueError("d must be a multiple of 32")
    blocks = X.reshape(-1, MX_BLOCK)
    E = mx_scale_exponents(np.max(np.abs(blocks), axis=1))
    codes = e4m3_round(np.ldexp(blocks, -E[:, None]))  # x / 2^E, exact in binary64
    scales = (E + 127).astype(np.uint8)
    return codes.reshape(X.shape), scales.reshape(X.shape[:-1] + (d // MX_BLOCK,))


def mx_dequantize(codes, scales) -> np.ndarray:
    """float64 values codes * 2^(scale - 127), blocks of 32 along the last axis."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.int64)
    vals = e4m3_table()[codes]
    E = np.repeat(scales - 127, MX_BLOCK, axis=-1)
    return np.ldexp(vals, E)


def attend_mx(Q, K, V, layout, sel, scale: Optional[float] = None,
              rows: Optional[Sequence[Tuple[int, int, int]]] = None):
    """Attention (8) with Q and K replaced by their MXFP8 dequantised values (rows are
    quantised independently, so with `rows` only the heads they touch are quantised)."""
    if rows is None:
        return attend(mx_dequantize(*mx_quantize(Q)), mx_dequantize(*mx_quantize(K)), V, layout,
                      sel, scale=scale)
    rows = list(rows)
    Q, K = _as_f64(Q), _as_f64(K)
    Qd = np.zeros_like(Q)
    Kd = np.zeros_like(K)
    for b, h in sorted({(b, h) for b, h, _ in rows}):
        Kd[b, h] = mx_dequantize(*mx_quantize(K[b, h]))
    for b, h, t in rows:
        Qd[b, h, t] = mx_dequantize(*mx_quantize(Q[b, h, t]))
    return attend(Qd, Kd, V, layout, sel, scale=scale, rows=rows)


# ---------------------------------------------------------------------------------------------
# 13. Quantised values: MXFP8 V along the key axis
# ---------------------------------------------------------------------------------------------
# Readings. In P.V the sum runs over keys, so a shared scale can only be factored out of the sum
# if it is shared along the keys: V is quantised with the rule of section 12 applied to each
# (b, h, dim) column, in blocks of 32 consecutive keys starting at key 0 (keys 32j .. 32j+31;
# the last block of a column is padded with zeros, which do not change its largest magnitude).
# The weights P are not part of the format: a kernel that rounds them to e4m3 before the
# product adds an error that pv_fp8_bound() bounds; attend_mxv() is the exact attention of the
# dequantised tensors.

def mx_quantize_keys(V) -> Tuple[np.ndarray, np.ndarray]:
    """MXFP8 of V [..., L, d] along the key axis: codes uint8 [..., d, L32] and E8M0 scale codes
    uint8 [..., d, L32/32], L32 = L rounded up to a multiple of 32 (padding keys are zero)."""
    V = _as_f64(V)
    L = V.shape[-2]
    L32 = -(-L // MX_BLOCK) * MX_BLOCK
    cols = np.zeros(V.shape[:-2] + (V.shape[-1], L32))
    cols[..., :L] = np.swapaxes(V, -1, -2)
    return mx_quantize(cols)


def mx_dequantize_keys(codes, scales, L: int) -> np.ndarray:
    """float64 V' [..., L, d] from the column codes and scales of mx_quantize_keys."""
    cols = mx_dequantize(codes, scales)
    return np.swapaxes(cols[..., :L], -1, -2)


def attend_mxv(Q, K, V, layout, sel, scale: Optional[float] = None,
               rows: Optional[Sequence[Tuple[int, int, int]]] = None):
    """Attention (8) over the dequantised Q', K' (rows along d, section 12) and V' (columns along
    the keys), in exact arithmetic."""
    V = _as_f64(V)
    Vd = mx_dequantize_keys(*mx_quantize_keys(V), V.shape[-2])
    return attend_mx(Q, K, Vd, layout, sel, scale=scale, rows=rows)


def pv_fp8_bound(Q, K, V, layout, sel, rows: Sequence[Tuple[int, int, int]],
                 scale: Optional[float] = None) -> np.ndarray:
    """Bound [n, d] on |o - o'| for the listed rows, where o is the attention (8) of Q, K, V
    (pass the dequantised tensors) and o' the same sum with every softmax weight rounded to
    e4m3 before it multiplies V.

    Derivation. With x_j the scaled scores of Omega(t), m = max x_j and p_j = exp(x_j - m), a
    kernel holds the weights as w_j = 2^delta p_j for some delta >= 0 of its own (a running
    maximum that trails the true one; delta <= 8 keeps w_j below the e4m3 maximum) and divides
    by its row sum 2^delta sum_j p_j of the unrounded weights. Rounding to nearest e4m3 moves a
    normal value (w >= 2^-6) by at most 2^-4 w, and a subnormal one by at most 2^-10 and at most
    w itself. The row error is therefore at most
        2^-4 sum_j p_j |v_j| / l  +  sum_j min(2^-10, p_j) |v_j| / l,    l = sum_j p_j,
    since 2^-delta min(2^-10, 2^delta p_j) <= min(2^-10, p_j). A row split into parts that are
    normalised separately and merged with their softmax weights obeys the same bound (each part's
    maximum is at most m, which only lowers its terms)."""
    D = derive(layout)
    Q, K, V = _as_f64(Q), _as_f64(K), _as_f64(V)
    d = Q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    sel = np.asarray(sel)
    out = np.zeros((len(rows), d))
    for i, (b, h, t) in enumerate(rows):
        keys = key_set(D, t, sel[b, h, t])
        x = (K[b, h][keys] @ Q[b, h, t]) * scale
        p = np.exp(x - np.max(x))
        av = np.abs(V[b, h][keys])
        out[i] = (2.0 ** -4 * (p @ av) + np.minimum(2.0 ** -10, p) @ av) / np.sum(p)
    return out


def _as_f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to(torch.float64).cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)
