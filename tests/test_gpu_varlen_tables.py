"""The work tables of the index inversion, element by element, through the C ABI.

moc_build_varlen lays out three tile lists besides the buckets and slots (jxzklqfsx.com write-up
of the MoC paper, section 計算效率: boundary tables from prefix sums, every (query group, key
group) pair packed into one variable-length problem):
* routed tiles (bucket, first position): ceil(n / tile_rows) per bucket of n routed rows, the
  buckets in (b, h, chunk) order;
* anchor tiles (query range, text range, own-shot range): the text queries first, then the
  queries of each shot (a maximal run of chunks with one shot id), tile_rows queries each;
* backward key tiles (key range, chunk or -1, query range, text split or -1): the text keys
  against each non-empty query split, then each shot chunk's keys against its own shot.
Here the expected lists are written out from those definitions in plain Python and compared
whole with what the GPU wrote, together with the tile counts and the int64 pair counts."""
import math

import numpy as np
import pytest
import torch

import moc_inputs as mi
from oracle import moc_oracle as mo
from test_gpu_parity import _say

pytestmark = pytest.mark.gpu


def _gpu_tables(w: mi.Workload):
    import sparse_chunk_routed_amd as moc
    dev = torch.device("cuda:0")
    Q, K, _ = mi.make_qkv(w)
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    cfg = moc.RouteCfg(w.top_k, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed)
    Qd, Kd = Q.to(dev), K.to(dev)
    kbar = moc.pool_keys(Kd, lay)
    sel, nsel = moc.route(Qd, kbar, lay, cfg)
    vl = moc.build_varlen(sel, nsel, lay, cfg, w.d, Qd.dtype)
    torch.cuda.synchronize()
    s = vl.struct
    n_r, n_a = vl.n_rtiles(), vl.n_atiles()
    n_k = int(vl._view(s.n_ktiles, 1).item())
    return dict(
        xcd_lo=vl._view(s.n_atiles, 10).cpu().numpy()[1:].astype(np.int64),
        sel=sel.cpu().numpy(), nsel=nsel.cpu().numpy(), BM=int(s.tile_rows),
        n_split=int(s.n_text_split), bucket_off=vl.bucket_off().cpu().numpy(),
        rtiles=vl._view(s.rtiles, 2 * n_r).cpu().numpy().reshape(-1, 2),
        atiles=vl._view(s.atiles, 6 * n_a).cpu().numpy().reshape(-1, 6),
        ktiles=vl._view(s.ktiles, 6 * n_k).cpu().numpy().reshape(-1, 6),
        pairs=vl.pair_count.cpu().numpy(),
        max=(int(s.max_rtiles), int(s.max_atiles), int(s.max_ktiles)))


def _shot_runs(lay: mi.Layout):
    """(first chunk, end chunk) of every maximal run of chunks with one shot id >= 0."""
    runs, c = [], 0
    while c < lay.C:
        sh = int(lay.chunk_shot[c])
        if sh < 0:
            c += 1
            continue
        c0 = c
        while c < lay.C and int(lay.chunk_shot[c]) == sh:
            c += 1
        runs.append((c0, c))
    return runs


def _expected(w: mi.Workload, g, KR: int):
    lay, BM = w.layout, g["BM"]
    off = [int(x) for x in lay.chunk_offsets]
    tb, te = lay.text_begin, lay.text_end
    B, H, Lq, S = g["sel"].shape
    # bucket sizes: how many (query, selection) entries name each chunk
    sizes = np.zeros((B, H, lay.C), np.int64)
    taken = np.arange(S)[None, None, None, :] < g["nsel"][..., None]
    for b in range(B):
        for h in range(H):
            sizes[b, h] = np.bincount(g["sel"][b, h][taken[b, h]].astype(np.int64),
                                      minlength=lay.C)
    flat = sizes.reshape(-1)
    bucket_off = np.concatenate([[0], np.cumsum(flat)])
    rtiles = [(i, k * BM) for i in range(flat.size) for k in range(-(-int(flat[i]) // BM))]
    groups = ([(tb, te, True)] if te > tb else []) + \
        [(off[c0], off[c1], False) for (c0, c1) in _shot_runs(lay)]
    atiles = []
    for q0, q1, text in groups:
        for q in range(q0, q1, BM):
            atiles.append((q, min(q + BM, q1), tb, te, 0 if text else q0, 0 if text else q1))
    ktiles = []
    if te > tb:
        qs = -(-lay.L // g["n_split"])
        splits = [sp for sp in range(g["n_split"]) if sp * qs < lay.L]
        for k0 in range(tb, te, KR):
            for sp in splits:
                ktiles.append((k0, min(k0 + KR, te), -1, sp * qs, min(sp * qs + qs, lay.L), sp))
    shot_range = {}
    for c0, c1 in _shot_runs(lay):
        for c in range(c0, c1):
            shot_range[c] = (off[c0], off[c1])
    for c in range(lay.C):
        if int(lay.chunk_shot[c]) < 0:
            continue
        for k0 in range(off[c], off[c + 1], KR):
            ktiles.append((k0, min(k0 + KR, off[c + 1]), c) + shot_range[c] + (-1,))
    return bucket_off, np.array(rtiles, np.int64).reshape(-1, 2), \
        np.array(atiles, np.int64).reshape(-1, 6), np.array(ktiles, np.int64).reshape(-1, 6)


def _xcd_ranges(atiles: np.ndarray, B: int, H: int, max_atiles: int) -> np.ndarray:
    """The 9 starts of the 8 anchor ranges, from their definition: item (b, h, tile) costs the
    tile's 64-key tiles (over its text range and its own-shot range) plus 4; range x starts at
    the first item whose cost prefix reaches x / 8 of the total, then kept monotone and within
    ceil(1.25 B H max_atiles / 8) items per range (and so that the later ranges can hold the
    rest)."""
    def k64(a, b):
        return ((b - 1) >> 6) - (a >> 6) + 1 if b > a else 0
    cost = np.array([k64(t[2], t[3]) + k64(t[4], t[5]) + 4 for t in atiles], np.int64)
    items = np.tile(cost, B * H)
    n = len(items)
    pref = np.concatenate([[0], np.cumsum(items)])
    slots = (B * H * max_atiles * 5 // 4 + 7) // 8
    lo = [0]
    for x in range(1, 8):
        v = int(np.searchsorted(pref, pref[-1] * x // 8, side="left")) if n else 0
        v = min(max(v, lo[-1], n - (8 - x) * slots), lo[-1] + slots, n)
        lo.append(v)
    lo.append(n)
    return np.array(lo, np.int64)


def _check(w: mi.Workload):
    g = _gpu_tables(w)
    kt = g["ktiles"]
    # the key rows per backward tile: the longest key tile (when every chunk and the text are
    # shorter, each is one tile whatever the key rows are)
    KR = int((kt[:, 1] - kt[:, 0]).max()) if len(kt) else 1
    bo, rt, at, kt_exp = _expected(w, g, KR)
    _say(f"{w.name}: L={w.L} C={w.C} B={w.B} H={w.H} tile_rows={g['BM']} key_rows={KR} "
         f"splits={g['n_split']} routed tiles {len(rt)} anchor tiles {len(at)} "
         f"key tiles {len(kt_exp)}")
    assert np.array_equal(g["bucket_off"], bo)
    assert np.array_equal(g["rtiles"], rt)
    assert np.array_equal(g["atiles"], at)
    assert np.array_equal(g["ktiles"], kt_exp)
    assert len(rt) <= g["max"][0] and len(at) <= g["max"][1] and len(kt_exp) <= g["max"][2]
    assert np.array_equal(g["pairs"], mo.pair_counts(w.layout, g["sel"]))
    xr = _xcd_ranges(at, w.B, w.H, g["max"][1])
    assert np.array_equal(g["xcd_lo"], xr), (g["xcd_lo"], xr)
    _say(f"anchor items per XCD range: {np.diff(xr).tolist()}")


@pytest.mark.parametrize("seed", range(6))
def test_tables_random_layouts(seed):
    """Irregular chunks, text first, last or absent, frame-is-shot (one group per chunk),
    B = 2, k from 0 to all chunks."""
    rng = np.random.default_rng(2000 + seed)
    lay = mi.make_random_layout(rng, max_shots=6, max_frames=5, max_chunk=700,
                                frame_is_shot=seed in (2, 5))
    top_k = min(lay.C, [2, 0, 3, lay.C, 1, 4][seed])
    w = mi.Workload(f"tables{seed}", 2, 3, 64, "bf16", lay, top_k=top_k, causal=seed != 3,
                    clustered_keys=True, seed=seed)
    _check(w)


def test_tables_max_chunks():
    """C = 1,024: 32 text tokens and 1,023 chunks of 16 tokens in 33 shots, top-k 32 with
    drop-in (1,024 chunks fill the one-workgroup scans over the layout exactly)."""
    sizes = [32] + [16] * 1023
    shots = [-1] + [i // 31 for i in range(1023)]
    lay = mi.layout_from_chunks(sizes, shots)
    w = mi.Workload("tables_maxc", 1, 2, 64, "bf16", lay, top_k=32, causal=True,
                    clustered_keys=True, p_max=0.5, lam=4.0, max_drop_in=16, seed=7)
    _check(w)


def test_tables_frame_is_shot_max_chunks():
    """1,024 one-chunk shots, no text: 1,024 anchor groups."""
    lay = mi.layout_from_chunks([40] * 1024, list(range(1024)))
    w = mi.Workload("tables_1024_shots", 1, 1, 64, "bf16", lay, top_k=3, causal=False,
                    clustered_keys=True, seed=3)
    _check(w)


def test_tables_headline():
    """The headline layout (175,232 tokens, 12 heads, 1,356 buckets, 11 text splits)."""
    w = mi.headline()
    _check(w)
    assert math.ceil(w.L / 16384) == 11
