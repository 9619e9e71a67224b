"""Seeded synthetic workloads for the Mixture-of-Contexts (MoC) attention layer.

This module is the ONLY code shared by the CPU oracle (``oracle/``) and the HIP path
(``sparse_chunk_routed_amd``). It builds token layouts (text range, frames, shots) and draws
random tensors; it contains none of the layer's arithmetic (no pooling, scoring, routing,
masking or attention).

Shapes follow the workloads the MoC pages describe: a caption (text) prefix followed by
frame-aligned video chunks grouped into shots (Mixture of Contexts summary, §3.2 "Attention
Chunking and Routing"; §4 "Experiments": 8 shots x 8 s, 480p, 12 fps, about 180k tokens), and a
latent frame of 30 x 52 = 1,560 patches. The actual LCT activations are not available, so seeded
normal tensors stand in for them; keys are clustered per chunk so that chunk descriptors differ
(the jxzklqfsx.com write-up, section "實驗 / 定性結果", notes that the tokens of one chunk are
highly redundant).

Random streams (numpy.random.default_rng): layout=seed, Q=seed+1, K centres=seed+2,
K noise=seed+3, V=seed+4, dO=seed+5. Tensors are drawn in fp32 and rounded to bf16 with
round-to-nearest-even (torch CPU ``.to(torch.bfloat16)``) when the workload is bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Optional, Sequence, Tuple

import numpy as np

FRAME_TOKENS = 1560  # 30 x 52 latent patch grid per latent frame


@dataclass(frozen=True)
class Layout:
    """Token layout of one sequence (shared by every batch element and head).

    chunk_offsets: int32 [C+1], 0 = off[0] < off[1] < ... < off[C] = L.
    chunk_shot:    int32 [C], shot id of each chunk; every text chunk carries -1. A shot's
                   chunks are contiguous.
    text_begin, text_end: the text tokens [t0, t1), a union of whole chunks (may be empty).
    """

    chunk_offsets: np.ndarray
    chunk_shot: np.ndarray
    text_begin: int
    text_end: int

    @property
    def L(self) -> int:
        return int(self.chunk_offsets[-1])

    @property
    def C(self) -> int:
        return int(len(self.chunk_shot))


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    dtype: str  # "f32" or "bf16"
    layout: Layout
    top_k: int
    causal: bool
    clustered_keys: bool
    p_max: float = 0.0
    lam: float = 0.0
    max_drop_in: int = 8
    seed: int = 0
    description: str = ""
    segments: Optional[Tuple[int, ...]] = None  # outer-loop routing: segment chunk offsets
    outer_M: int = 0
    mx_scores: bool = False  # quantised scores: Q and K as MXFP8 in the attention
    mx_values: bool = False  # quantised values: V as MXFP8 along the keys, P.V on fp8 as well

    @property
    def L(self) -> int:
        return self.layout.L

    @property
    def C(self) -> int:
        return self.layout.C


def build_layout(text_tokens: int, shot_frames: Sequence[int], frame_tokens: int,
                 text_first: bool = True, frame_is_shot: bool = False) -> Layout:
    """Text chunk (one chunk, if any) plus one chunk per frame; frames grouped into shots.

    frame_is_shot gives every frame its own shot id (single-shot clips whose mandatory local
    link is the query's own chunk)."""
    sizes: List[int] = []
    shots: List[int] = []
    video_sizes: List[int] = []
    video_shots: List[int] = []
    sid = 0
    for nf in shot_frames:
        for _ in range(int(nf)):
            video_sizes.append(int(frame_tokens))
            video_shots.append(sid)
            if frame_is_shot:
                sid += 1
        if not frame_is_shot:
            sid += 1
    if text_tokens > 0 and text_first:
        sizes.append(int(text_tokens))
        shots.append(-1)
    sizes += video_sizes
    shots += video_shots
    if text_tokens > 0 and not text_first:
        sizes.append(int(text_tokens))
        shots.append(-1)
    off = np.zeros(len(sizes) + 1, dtype=np.int32)
    off[1:] = np.cumsum(sizes)
    if text_tokens > 0:
        tb = 0 if text_first else int(off[-2])
        te = tb + int(text_tokens)
    else:
        tb = te = 0
    return Layout(off, np.asarray(shots, dtype=np.int32), tb, te)


def layout_from_chunks(chunk_sizes: Sequence[int], chunk_shot: Sequence[int]) -> Layout:
    """General layout from explicit chunk sizes and shot ids (-1 = text).

    All text chunks must be contiguous."""
    off = np.zeros(len(chunk_sizes) + 1, dtype=np.int32)
    off[1:] = np.cumsum(np.asarray(chunk_sizes, dtype=np.int64))
    shots = np.asarray(chunk_shot, dtype=np.int32)
    tidx = np.nonzero(shots < 0)[0]
    if len(tidx) == 0:
        tb = te = 0
    else:
        if not np.all(np.diff(tidx) == 1):
            raise ValueError("text chunks must be contiguous")
        tb, te = int(off[tidx[0]]), int(off[tidx[-1] + 1])
    return Layout(off, shots, tb, te)


def irregular_shot_frames(seed: int, n_shots: int = 8, total: int = 112,
                          lo: int = 10, hi: int = 18) -> List[int]:
    """Frames per shot drawn uniform in [lo, hi], rescaled to sum to `total` by the largest
    remainder method (ties go to the lower shot index). Rescaled sizes may fall outside
    [lo, hi]; that is accepted."""
    rng = np.random.default_rng(seed)
    raw = rng.integers(lo, hi + 1, size=n_shots).astype(np.int64)
    # exact rational shares raw_i * total / sum(raw)
    s = int(raw.sum())
    num = raw * total
    base = num // s
    rem = num - base * s
    short = total - int(base.sum())
    order = sorted(range(n_shots), key=lambda i: (-int(rem[i]), i))
    out = base.copy()
    for i in order[:short]:
        out[i] += 1
    assert int(out.sum()) == total
    return [int(x) for x in out]


# ---------------------------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------------------------

def tiny(seed: int = 0, **kw) -> Workload:
    """fp32, B=1 H=2 d=64; 128 text tokens + 4 shots x 4 frames x 256 tokens = 4,224 tokens;
    C=17; top_k=2, causal; Q, K, V ~ N(0,1)."""
    lay = build_layout(128, [4, 4, 4, 4], 256)
    w = Workload("tiny", 1, 2, 64, "f32", lay, top_k=2, causal=True, clustered_keys=False,
                 seed=seed, description="128 text + 4 shots x 4 frames x 256 tokens")
    return replace(w, **kw)


def mid(seed: int = 0, **kw) -> Workload:
    """bf16, B=1 H=12 d=128; 512 text + 8 shots x 8 frames x 1,560 = 100,352 tokens; C=65;
    top_k=4, causal; clustered keys."""
    lay = build_layout(512, [8] * 8, FRAME_TOKENS)
    w = Workload("mid", 1, 12, 128, "bf16", lay, top_k=4, causal=True, clustered_keys=True,
                 seed=seed, description="512 text + 8 shots x 8 frames x 1560 tokens")
    return replace(w, **kw)


def headline(seed: int = 0, **kw) -> Workload:
    """bf16, B=1 H=12 d=128; 512 text + 112 frames x 1,560 in 8 irregular shots = 175,232
    tokens; C=113; top_k=2 (the largest k leaving >= 85% of pairs pruned for seeds 0-7;
    checked by the oracle tests); causal; clustered keys."""
    frames = irregular_shot_frames(seed)
    lay = build_layout(512, frames, FRAME_TOKENS)
    w = Workload("headline", 1, 12, 128, "bf16", lay, top_k=2, causal=True,
                 clustered_keys=True, seed=seed,
                 description="512 text + 112 frames x 1560 tokens in 8 irregular shots "
                             f"(frames per shot {frames})")
    return replace(w, **kw)


def headline_uniform(seed: int = 0, **kw) -> Workload:
    lay = build_layout(512, [14] * 8, FRAME_TOKENS)
    w = Workload("headline_uniform", 1, 12, 128, "bf16", lay, top_k=2, causal=True,
                 clustered_keys=True, seed=seed,
                 description="512 text + 8 shots x 14 frames x 1560 tokens")
    return replace(w, **kw)


def short(seed: int = 0, **kw) -> Workload:
    """bf16, B=1 H=12 d=128; 256 text + 21 frames x 1,560 = 33,016 tokens; each frame is its
    own shot (mandatory links: text + own frame); top_k=3, causal; clustered keys."""
    lay = build_layout(256, [21], FRAME_TOKENS, frame_is_shot=True)
    w = Workload("short", 1, 12, 128, "bf16", lay, top_k=3, causal=True, clustered_keys=True,
                 seed=seed, description="256 text + 21 frames x 1560 tokens, frame = shot")
    return replace(w, **kw)


def train(seed: int = 0, **kw) -> Workload:
    """Headline layout with training-time routing noise: drop-off p ~ U(0, 0.3), drop-in
    m ~ Poisson(1) capped at 8."""
    w = headline(seed)
    w = replace(w, name="train", p_max=0.3, lam=1.0, max_drop_in=8,
                description=w.description + "; drop-off p_max=0.3, drop-in lambda=1")
    return replace(w, **kw)


def grad_slice(seed: int = 0, **kw) -> Workload:
    """The 4,224-token gradient slice: the tiny layout at the headline head shape (H=12,
    d=128), bf16, top_k=2, causal, p_max=0.3, lambda=1."""
    lay = build_layout(128, [4, 4, 4, 4], 256)
    w = Workload("slice", 1, 12, 128, "bf16", lay, top_k=2, causal=True, clustered_keys=True,
                 p_max=0.3, lam=1.0, max_drop_in=8, seed=seed,
                 description="128 text + 4 shots x 4 frames x 256 tokens, H=12 d=128")
    return replace(w, **kw)


def fixed_chunk_layout(text_tokens: int, visual_tokens: int, chunk: int) -> Layout:
    """Text chunk plus fixed-size visual chunks that ignore frame boundaries (the last one is
    ragged). Every visual chunk carries its own shot id, so a query's mandatory local link is its
    own chunk (the single-shot recipe: mandatory intra-chunk and text links, Mixture of Contexts
    summary, Appendix F)."""
    n = -(-int(visual_tokens) // int(chunk))
    sizes = ([int(text_tokens)] if text_tokens > 0 else []) + \
        [min(int(chunk), int(visual_tokens) - i * int(chunk)) for i in range(n)]
    shots = ([-1] if text_tokens > 0 else []) + list(range(n))
    return layout_from_chunks(sizes, shots)


SINGLE_SHOT_FRAMES = 24        # 8 s at 12 fps, 4x temporal latent compression
SINGLE_SHOT_FRAME_TOKENS = 252  # 320 x 192 clip: 256 text + 24 x 252 = 6,304 tokens (~6,300)


def single_shot(seed: int = 0, chunk: int = 256, **kw) -> Workload:
    """Single-shot short clip with fixed-size chunks (Mixture of Contexts summary, Appendix E-G
    and Table 3: about 6,300 tokens, chunk size 256, top-k 3, intra-chunk and text links, no
    causal routing; Table 3 sweeps chunk sizes 64 to 1024). bf16, B=1 H=12 d=128."""
    lay = fixed_chunk_layout(256, SINGLE_SHOT_FRAMES * SINGLE_SHOT_FRAME_TOKENS, chunk)
    w = Workload(f"single_shot_c{chunk}", 1, 12, 128, "bf16", lay, top_k=3, causal=False,
                 clustered_keys=True, seed=seed,
                 description=(f"256 text + 24 frames x 252 tokens in fixed {chunk}-token chunks, "
                              "chunk = shot, non-causal"))
    return replace(w, **kw)


def shots(seed: int = 0, n_shots: int = 8, frames_per_shot: int = 14, **kw) -> Workload:
    """Multi-shot sequence for the length sweep: 512 text + n_shots x frames_per_shot frames of
    1,560 tokens (14 frames = 21,840 tokens, the headline's mean shot), top_k=2, causal."""
    lay = build_layout(512, [frames_per_shot] * n_shots, FRAME_TOKENS)
    w = Workload(f"shots{n_shots}", 1, 12, 128, "bf16", lay, top_k=2, causal=True,
                 clustered_keys=True, seed=seed,
                 description=f"512 text + {n_shots} shots x {frames_per_shot} frames x 1560 tokens")
    return replace(w, **kw)


def dense(seed: int = 0, n_shots: int = 8, frames_per_shot: int = 14, **kw) -> Workload:
    """Dense attention over the same token count as shots(n_shots): one shot holding every token
    and no text range, so every query attends every key (no routing, top_k=0)."""
    L = 512 + n_shots * frames_per_shot * FRAME_TOKENS
    sizes = [512] + [FRAME_TOKENS] * (n_shots * frames_per_shot)
    lay = layout_from_chunks(sizes, [0] * len(sizes))
    assert lay.L == L
    w = Workload(f"dense{n_shots}", 1, 12, 128, "bf16", lay, top_k=0, causal=True,
                 clustered_keys=True, seed=seed,
                 description=f"dense attention over {L} tokens (one shot, no routing)")
    return replace(w, **kw)


def shot_segments(layout: Layout) -> Tuple[int, ...]:
    """Segment chunk offsets with one segment per shot (the text chunks form one segment)."""
    shot = list(layout.chunk_shot)
    cuts = [0] + [c for c in range(1, len(shot)) if shot[c] != shot[c - 1]] + [len(shot)]
    return tuple(cuts)


def headline_outer(seed: int = 0, **kw) -> Workload:
    """Headline layout with outer-loop context routing: one segment per shot (and the text),
    each query segment picks its top-2 earlier shots, and inner top-2 routing runs only within
    the query's own shot segment and those two."""
    w = headline(seed)
    w = replace(w, name="headline_outer", segments=shot_segments(w.layout), outer_M=2,
                description=w.description + "; outer routing over shots, M=2")
    return replace(w, **kw)


def headline_h3(seed: int = 0, **kw) -> Workload:
    """One GPU's share of the headline layer sharded four ways by head: H=3 at the full
    175,232-token layout (routing and attention are independent per head)."""
    w = headline(seed)
    w = replace(w, name="headline_h3", H=3,
                description=w.description + "; 3 of 12 heads (a 4-way head shard)")
    return replace(w, **kw)


def headline_mx(seed: int = 0, **kw) -> Workload:
    """Headline workload with quantised scores: Q and K quantised to MXFP8 for the attention
    (routing and pooling on the bf16 inputs as before), V and P.V in bf16."""
    w = headline(seed)
    w = replace(w, name="headline_mx", mx_scores=True,
                description=w.description + "; attention scores from MXFP8 Q and K")
    return replace(w, **kw)


def headline_mxv(seed: int = 0, **kw) -> Workload:
    """Headline workload with quantised scores and values: Q, K and V quantised to MXFP8 for the
    attention (V in 32-key blocks), P.V on fp8 with the softmax weights rounded to e4m3."""
    w = headline(seed)
    w = replace(w, name="headline_mxv", mx_scores=True, mx_values=True,
                description=w.description + "; attention from MXFP8 Q, K and V")
    return replace(w, **kw)


WORKLOADS = {"tiny": tiny, "mid": mid, "headline": headline, "short": short, "train": train,
             "slice": grad_slice, "headline_uniform": headline_uniform,
             "single_shot": single_shot, "headline_outer": headline_outer,
             "headline_mx": headline_mx, "headline_mxv": headline_mxv,
             "headline_h3": headline_h3}
for _c in (64, 128, 256, 512, 1024):
    WORKLOADS[f"single_shot_c{_c}"] = (lambda c: lambda seed=0, **kw: single_shot(seed, c, **kw))(_c)


# ---------------------------------------------------------------------------------------------
# Tensors
# ---------------------------------------------------------------------------------------------

def _round_dtype(x: np.ndarray, dtype: str):
    """fp32 numpy array -> torch CPU tensor in the workload dtype (RNE for bf16)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(dtype)


def chunk_sizes(layout: Layout) -> np.ndarray:
    return np.diff(layout.chunk_offsets.astype(np.int64))


def make_qkv(w: Workload, with_dout: bool = False):
    """Seeded Q, K, V (and dO) as torch CPU tensors [B,H,L,d] in the workload dtype."""
    B, H, L, d = w.B, w.H, w.L, w.d
    s = w.seed
    q = np.random.default_rng(s + 1).standard_normal((B, H, L, d), dtype=np.float32)
    Q = _round_dtype(q, w.dtype)
    del q
    if w.clustered_keys:
        C = w.C
        centres = np.random.default_rng(s + 2).standard_normal((B, H, C, d), dtype=np.float32)
        noise = np.random.default_rng(s + 3).standard_normal((B, H, L, d), dtype=np.float32)
        reps = chunk_sizes(w.layout)
        k = np.repeat(centres, reps, axis=2)
        k += np.float32(0.5) * noise
        del noise
    else:
        k = np.random.default_rng(s + 3).standard_normal((B, H, L, d), dtype=np.float32)
    K = _round_dtype(k, w.dtype)
    del k
    v = np.random.default_rng(s + 4).standard_normal((B, H, L, d), dtype=np.float32)
    V = _round_dtype(v, w.dtype)
    del v
    if not with_dout:
        return Q, K, V
    g = np.random.default_rng(s + 5).standard_normal((B, H, L, d), dtype=np.float32)
    dO = _round_dtype(g, w.dtype)
    return Q, K, V, dO


def make_random_layout(rng: np.random.Generator, max_shots: int = 5, max_frames: int = 4,
                       max_chunk: int = 40, text: Optional[int] = None,
                       text_first: Optional[bool] = None, frame_is_shot: bool = False) -> Layout:
    """Random small layout with irregular chunk sizes, for property tests."""
    n_shots = int(rng.integers(1, max_shots + 1))
    if text is None:
        text = int(rng.integers(0, 3)) * int(rng.integers(1, max_chunk + 1))
    if text_first is None:
        text_first = bool(rng.integers(0, 2))
    sizes: List[int] = []
    shots: List[int] = []
    sid = 0
    for _ in range(n_shots):
        nf = int(rng.integers(1, max_frames + 1))
        for _ in range(nf):
            sizes.append(int(rng.integers(1, max_chunk + 1)))
            shots.append(sid)
            if frame_is_shot:
                sid += 1
        if not frame_is_shot:
            sid += 1
    if text > 0:
        if text_first:
            sizes.insert(0, text)
            shots.insert(0, -1)
        else:
            sizes.append(text)
            shots.append(-1)
    return layout_from_chunks(sizes, shots)
