"""Python surface of libmoc: the C-ABI entry points with the same names, taking torch tensors.

torch supplies device memory and the current HIP stream; every step of the layer runs in the
library's HIP kernels. Nothing here computes any part of the layer.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib as L


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return L.MOC_BF16
    if dt == torch.float32:
        return L.MOC_F32
    raise TypeError(f"unsupported dtype {dt} (bfloat16 or float32)")


class DeviceLayout:
    """A token layout resident on the device: chunk offsets [C+1], chunk shot ids [C]
    (-1 = text) and the text range. The content is validated here on the host copy, since the
    library treats it as a precondition. With device_check=True the library also checks it on
    the device at the start of every call (moc_layout.check): the word lives in `check_word`
    and check_status() reads it."""

    def __init__(self, chunk_offsets: Sequence[int], chunk_shot: Sequence[int], text_begin: int,
                 text_end: int, device="cuda", device_check: bool = False,
                 validate: bool = True):
        off = np.asarray(chunk_offsets, dtype=np.int64)
        shot = np.asarray(chunk_shot, dtype=np.int64)
        if validate:
            validate_layout(off, shot, int(text_begin), int(text_end))
        self.C = int(len(shot))
        self.L = int(off[-1])
        self.text_begin, self.text_end = int(text_begin), int(text_end)
        self.offsets_host = off.astype(np.int32)
        self.shot_host = shot.astype(np.int32)
        self.offsets = torch.from_numpy(self.offsets_host.copy()).to(device)
        self.shot = torch.from_numpy(self.shot_host.copy()).to(device)
        self.check_word = (torch.zeros(1, dtype=torch.int32, device=device) if device_check
                           else None)

    def check_status(self) -> None:
        """Wait for the device, then raise MocError(MOC_ELAYOUT) if the check word is set."""
        if self.check_word is None:
            return
        word = int(self.check_word.item()) & 0xFFFFFFFF
        lib = L.load()
        L.check(lib.moc_layout_status(word))

    def check_on_device(self) -> None:
        """Enqueue only the layout check (moc_check_layout) on the current stream."""
        if self.check_word is None:
            raise ValueError("built without device_check")
        s = self.struct(1, 1, 64, torch.bfloat16)
        L.check(L.load().moc_check_layout(ctypes.byref(s), _stream(self.offsets.device)))

    @classmethod
    def from_layout(cls, lay, device="cuda") -> "DeviceLayout":
        return cls(lay.chunk_offsets, lay.chunk_shot, lay.text_begin, lay.text_end, device)

    def struct(self, B: int, H: int, d: int, dtype: torch.dtype) -> L.MocLayout:
        return L.MocLayout(B, H, self.L, d, _dtype_code(dtype), self.C, self.offsets.data_ptr(),
                           self.shot.data_ptr(), self.text_begin, self.text_end,
                           None if self.check_word is None else self.check_word.data_ptr())


def layout_check_host(off, shot, tb: int, te: int) -> int:
    """The library's layout check on host arrays (moc_layout_check_host): MOC_LAYOUT_* bits, 0
    for a valid layout."""
    o = np.ascontiguousarray(off, dtype=np.int32)
    sh = np.ascontiguousarray(shot, dtype=np.int32)
    return int(L.load().moc_layout_check_host(o.ctypes.data, sh.ctypes.data, len(sh),
                                               int(o[-1]), int(tb), int(te)))


def validate_layout(off: np.ndarray, shot: np.ndarray, tb: int, te: int) -> None:
    C = len(shot)
    if C < 1 or len(off) != C + 1 or off[0] != 0 or np.any(np.diff(off) <= 0):
        raise ValueError("chunk offsets must be 0 = off[0] < off[1] < ... < off[C]")
    if C > L.MOC_MAX_C:
        raise ValueError(f"at most {L.MOC_MAX_C} chunks")
    Ltot = int(off[-1])
    if not (0 <= tb <= te <= Ltot):
        raise ValueError("text range outside the sequence")
    seen, prev = set(), None
    for c in range(C):
        a, b = int(off[c]), int(off[c + 1])
        in_text = tb <= a and b <= te and tb < te
        if (a < te and tb < b) and not in_text:
            raise ValueError(f"chunk {c} straddles the text range")
        if in_text != (shot[c] == -1):
            raise ValueError(f"chunk {c}: text chunks carry shot -1, and only they")
        s = int(shot[c])
        if s == -1:
            prev = None
            continue
        if s < 0:
            raise ValueError("shot ids must be >= 0 (or -1 for text)")
        if s != prev:
            if s in seen:
                raise ValueError(f"shot {s} is not contiguous")
            seen.add(s)
        prev = s
    if tb < te:
        idx = np.nonzero(shot == -1)[0]
        if int(off[idx[0]]) != tb or int(off[idx[-1] + 1]) != te:
            raise ValueError("text range must be a union of whole chunks")


@dataclass
class RouteCfg:
    top_k: int
    causal: bool = True
    p_max: float = 0.0
    lam: float = 0.0
    max_drop_in: int = 8
    seed: int = 0

    def struct(self) -> L.MocRouteCfg:
        return L.MocRouteCfg(int(self.top_k), 1 if self.causal else 0, float(self.p_max),
                             float(self.lam), int(self.max_drop_in), 0,
                             int(self.seed) & ((1 << 64) - 1))


def _check_qkv(*ts: torch.Tensor) -> None:
    t0 = ts[0]
    for t in ts:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B,H,L,d]")
        if t.shape != t0.shape or t.dtype != t0.dtype:
            raise ValueError("Q/K/V-like tensors must share shape and dtype")


def sel_width(cfg: RouteCfg, C: int) -> int:
    lib = L.load()
    return int(lib.moc_sel_width(ctypes.byref(cfg.struct()), C))


def workspace_bytes(lay: DeviceLayout, B: int, H: int, d: int, dtype: torch.dtype,
                    cfg: RouteCfg, op: int) -> int:
    lib = L.load()
    s = lay.struct(B, H, d, dtype)
    n = int(lib.moc_workspace_bytes(ctypes.byref(s), ctypes.byref(cfg.struct()), op))
    if n == 0 and op != L.MOC_OP_ROUTE:
        raise L.MocError(L.MOC_EINVAL, lib.moc_last_error().decode())
    return n


def pool_keys(K: torch.Tensor, lay: DeviceLayout) -> torch.Tensor:
    """kbar [B,H,C,d] fp32: the mean of each chunk's keys."""
    _check_qkv(K)
    B, H, Lq, d = K.shape
    kbar = torch.empty((B, H, lay.C, d), dtype=torch.float32, device=K.device)
    s = lay.struct(B, H, d, K.dtype)
    lib = L.load()
    L.check(lib.moc_pool_keys(ctypes.byref(s), _ptr(K), _ptr(kbar), _stream(K.device)))
    return kbar


def route(Q: torch.Tensor, kbar: torch.Tensor, lay: DeviceLayout, cfg: RouteCfg,
          ws: Optional[torch.Tensor] = None, cand_mask: Optional[torch.Tensor] = None):
    """(sel [B,H,L,S] int32 ascending, -1 padded; nsel [B,H,L] int32). With cand_mask (the
    int32 view of the uint32 [B,H,C,ceil(C/32)] mask of route_outer), the inner router of
    outer-loop routing (moc_route_masked)."""
    _check_qkv(Q)
    B, H, Lq, d = Q.shape
    S = sel_width(cfg, lay.C)
    sel = torch.empty((B, H, Lq, S), dtype=torch.int32, device=Q.device)
    nsel = torch.empty((B, H, Lq), dtype=torch.int32, device=Q.device)
    s = lay.struct(B, H, d, Q.dtype)
    lib = L.load()
    need = workspace_bytes(lay, B, H, d, Q.dtype, cfg, L.MOC_OP_ROUTE)
    if need > 0 and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    args = (_ptr(sel) if S > 0 else None, _ptr(nsel), _ptr(ws) if need > 0 else None,
            ws.numel() if need > 0 else 0, _stream(Q.device))
    if cand_mask is None:
        L.check(lib.moc_route(ctypes.byref(s), ctypes.byref(cfg.struct()), _ptr(Q), _ptr(kbar),
                              *args))
    else:
        W = (lay.C + 31) // 32
        if (cand_mask.dtype != torch.int32 or tuple(cand_mask.shape) != (B, H, lay.C, W)
                or not cand_mask.is_contiguous() or cand_mask.device != Q.device):
            raise ValueError(f"cand_mask must be int32 [{B},{H},{lay.C},{W}] on {Q.device}")
        L.check(lib.moc_route_masked(ctypes.byref(s), ctypes.byref(cfg.struct()), _ptr(Q),
                                     _ptr(kbar), _ptr(cand_mask), *args))
    return sel, nsel


@dataclass
class OuterRouting:
    seg_sel: torch.Tensor    # int32 [B,H,nseg,min(M,nseg)] ascending, -1 padded
    seg_nsel: torch.Tensor   # int32 [B,H,nseg]
    cand_mask: torch.Tensor  # int32 view of uint32 [B,H,C,ceil(C/32)]


class DeviceSegments:
    """Outer-routing segments resident on the device: chunk offsets [nseg+1] of groups of whole
    chunks. The content is validated here on the host copy against the layout (start at 0,
    increase strictly, end at C, no segment mixing text and video chunks), since the library
    treats it as a precondition; building one per layout keeps the routing call free of host
    copies and synchronisation."""

    def __init__(self, seg_chunk: Sequence[int], lay: DeviceLayout):
        h = [int(x) for x in np.asarray(seg_chunk, dtype=np.int64).ravel()]
        nseg = len(h) - 1
        if nseg < 1 or h[0] != 0 or h[-1] != lay.C or any(b <= a for a, b in zip(h, h[1:])):
            raise ValueError("seg_chunk must start at 0, increase strictly and end at C")
        if nseg > L.MOC_MAX_SEG:
            raise ValueError(f"at most {L.MOC_MAX_SEG} segments")
        for a, b in zip(h, h[1:]):
            kinds = {int(x) < 0 for x in lay.shot_host[a:b]}
            if len(kinds) != 1:
                raise ValueError(f"segment of chunks [{a}, {b}) mixes text and video chunks")
        self.host = h
        self.nseg = nseg
        self.C = lay.C
        self.dev = torch.tensor(h, dtype=torch.int32, device=lay.offsets.device)


def route_outer(Q: torch.Tensor, K: torch.Tensor, lay: DeviceLayout, seg_chunk, M: int,
                causal: bool, ws: Optional[torch.Tensor] = None) -> OuterRouting:
    """Outer-loop context routing (moc_route_outer): seg_chunk is a DeviceSegments or a host
    sequence of the segments' chunk offsets [nseg+1] (validated and uploaded per call)."""
    _check_qkv(Q)
    _check_qkv(K)
    B, H, Lq, d = Q.shape
    segs = seg_chunk if isinstance(seg_chunk, DeviceSegments) else DeviceSegments(seg_chunk, lay)
    if segs.C != lay.C or segs.dev.device != Q.device:
        raise ValueError("segments built for another layout or device")
    seg, nseg = segs.dev, segs.nseg
    Ms = min(int(M), nseg)
    W = (lay.C + 31) // 32
    seg_sel = torch.empty((B, H, nseg, Ms), dtype=torch.int32, device=Q.device)
    seg_nsel = torch.empty((B, H, nseg), dtype=torch.int32, device=Q.device)
    cmask = torch.empty((B, H, lay.C, W), dtype=torch.int32, device=Q.device)
    s = lay.struct(B, H, d, Q.dtype)
    need = workspace_bytes(lay, B, H, d, Q.dtype, RouteCfg(0, causal), L.MOC_OP_OUTER)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    lib = L.load()
    L.check(lib.moc_route_outer(ctypes.byref(s), _ptr(seg), nseg, int(M), int(bool(causal)),
                                _ptr(Q), _ptr(K), _ptr(seg_sel) if Ms > 0 else None,
                                _ptr(seg_nsel), _ptr(cmask), _ptr(ws), ws.numel(),
                                _stream(Q.device)))
    return OuterRouting(seg_sel, seg_nsel, cmask)


class Varlen:
    """The inverted index (per-chunk query buckets, slots, work tiles) and its workspace."""

    def __init__(self, struct: L.MocVarlen, ws: torch.Tensor, pair_count: torch.Tensor,
                 cfg: RouteCfg, lay: DeviceLayout, B: int, H: int, d: int = 128,
                 dtype: torch.dtype = torch.bfloat16):
        self.struct = struct
        self.ws = ws
        self.pair_count = pair_count
        self.cfg = cfg
        self.layout = lay
        self.B, self.H = B, H
        self.d, self.dtype = d, dtype

    @property
    def S(self) -> int:
        return int(self.struct.S)

    def _view(self, addr: int, n: int) -> torch.Tensor:
        base = self.ws.data_ptr()
        off = addr - base
        assert off % 4 == 0 and 0 <= off and off + 4 * n <= self.ws.numel()
        return self.ws[off:off + 4 * n].view(torch.int32)

    def bucket_off(self) -> torch.Tensor:
        return self._view(self.struct.bucket_off, self.B * self.H * self.layout.C + 1)

    def bucket_q(self, total: int) -> torch.Tensor:
        return self._view(self.struct.bucket_q, total)

    def slot(self, Lq: int) -> torch.Tensor:
        S = self.S
        return self._view(self.struct.slot, self.B * self.H * Lq * S).view(self.B, self.H, Lq, S)

    def n_rtiles(self) -> int:
        return int(self._view(self.struct.n_rtiles, 1).item())

    def n_atiles(self) -> int:
        return int(self._view(self.struct.n_atiles, 1).item())

    def _lay(self):
        return self.layout.struct(self.B, self.H, self.d, self.dtype)

    def total(self) -> int:
        """Total routed (query, chunk) rows of the routing (moc_varlen_total: waits for the
        current stream)."""
        t = ctypes.c_int64(0)
        s = self._lay()
        L.check(L.load().moc_varlen_total(ctypes.byref(s), ctypes.byref(self.struct),
                                          ctypes.byref(t), _stream(self.ws.device)))
        return int(t.value)

    def set_capacity(self, routed_cap: int) -> None:
        """Size the attention workspaces for `routed_cap` routed rows (moc_varlen_set_capacity);
        a capacity below total() makes the attention calls write nothing (check_status)."""
        L.check(L.load().moc_varlen_set_capacity(ctypes.byref(self.struct), int(routed_cap)))

    def workspace_bytes(self, op: int) -> int:
        """Bytes of the FWD or BWD workspace at the current capacity."""
        s = self._lay()
        n = int(L.load().moc_attend_workspace_bytes(ctypes.byref(s), ctypes.byref(self.struct),
                                                    op))
        if n == 0:
            raise L.MocError(L.MOC_EINVAL, L.load().moc_last_error().decode())
        return n

    def check_status(self) -> None:
        """Wait for the current stream; raise MocError if the last attention call found more
        routed rows than the capacity (MOC_EWORKSPACE) or a set layout check word."""
        L.check(L.load().moc_varlen_status(ctypes.byref(self.struct), _stream(self.ws.device)))


def build_varlen(sel: torch.Tensor, nsel: torch.Tensor, lay: DeviceLayout, cfg: RouteCfg,
                 d: int, dtype: torch.dtype) -> Varlen:
    B, H, Lq = nsel.shape
    ws_n = workspace_bytes(lay, B, H, d, dtype, cfg, L.MOC_OP_VARLEN)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=nsel.device)
    pair = torch.empty((B, H), dtype=torch.int64, device=nsel.device)
    vs = L.MocVarlen()
    s = lay.struct(B, H, d, dtype)
    lib = L.load()
    S = sel_width(cfg, lay.C)
    L.check(lib.moc_build_varlen(ctypes.byref(s), ctypes.byref(cfg.struct()),
                                 _ptr(sel) if S > 0 else None, _ptr(nsel), ctypes.byref(vs),
                                 _ptr(pair), _ptr(ws), ws_n, _stream(nsel.device)))
    return Varlen(vs, ws, pair, cfg, lay, B, H, d, dtype)


def attend_fwd(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, lay: DeviceLayout,
               vl: Varlen, scale: Optional[float] = None, ws: Optional[torch.Tensor] = None):
    """(O [B,H,L,d] in the input dtype, lse [B,H,L] fp32, natural log)."""
    _check_qkv(Q, K, V)
    B, H, Lq, d = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = torch.empty_like(Q)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=Q.device)
    need = vl.workspace_bytes(L.MOC_OP_FWD)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    s = lay.struct(B, H, d, Q.dtype)
    lib = L.load()
    L.check(lib.moc_attend_fwd(ctypes.byref(s), ctypes.byref(vl.struct), _ptr(Q), _ptr(K), _ptr(V),
                               float(scale), _ptr(O), _ptr(lse), _ptr(ws), ws.numel(),
                               _stream(Q.device)))
    return O, lse


@dataclass
class MxTensor:
    """MXFP8 rows of a [B,H,L,d] tensor (moc_mx_quantize): codes uint8 [B,H,Lp,d] and E8M0
    scales uint8 [B,H,Lp,d/32], rows padded to Lp = L rounded up to 64."""
    codes: torch.Tensor
    scales: torch.Tensor
    L: int


def mx_quantize(X: torch.Tensor, lay: DeviceLayout, out: Optional[MxTensor] = None) -> MxTensor:
    """MXFP8 quantisation of a bf16 [B,H,L,d] tensor (moc_mx_quantize)."""
    _check_qkv(X)
    if X.dtype != torch.bfloat16:
        raise ValueError("MXFP8 quantisation takes bf16 input")
    B, H, Lq, d = X.shape
    Lp = (Lq + 63) // 64 * 64
    if out is None or out.codes.shape != (B, H, Lp, d):
        out = MxTensor(torch.empty((B, H, Lp, d), dtype=torch.uint8, device=X.device),
                       torch.empty((B, H, Lp, d // 32), dtype=torch.uint8, device=X.device), Lq)
    s = lay.struct(B, H, d, X.dtype)
    L.check(L.load().moc_mx_quantize(ctypes.byref(s), _ptr(X), _ptr(out.codes), _ptr(out.scales),
                                     _stream(X.device)))
    return out


def attend_fwd_mx(Qm: MxTensor, Km: MxTensor, V: torch.Tensor, lay: DeviceLayout, vl: Varlen,
                  scale: Optional[float] = None, ws: Optional[torch.Tensor] = None):
    """Forward with quantised scores (moc_attend_fwd_mx): (O [B,H,L,d] bf16, lse [B,H,L])."""
    _check_qkv(V)
    B, H, Lq, d = V.shape
    Lp = (Lq + 63) // 64 * 64
    for m in (Qm, Km):
        if m.codes.shape != (B, H, Lp, d) or m.scales.shape != (B, H, Lp, d // 32):
            raise ValueError("MXFP8 operands do not match V's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = torch.empty_like(V)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=V.device)
    need = vl.workspace_bytes(L.MOC_OP_FWD)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=V.device)
    s = lay.struct(B, H, d, V.dtype)
    L.check(L.load().moc_attend_fwd_mx(ctypes.byref(s), ctypes.byref(vl.struct), _ptr(Qm.codes),
                                       _ptr(Qm.scales), _ptr(Km.codes), _ptr(Km.scales), _ptr(V),
                                       float(scale), _ptr(O), _ptr(lse), _ptr(ws), ws.numel(),
                                       _stream(V.device)))
    return O, lse


VQ_ROW = 80  # bytes per (64-key tile, dim) row of the quantised V tiles


def mx_quantize_v(V: torch.Tensor, lay: DeviceLayout,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """MXFP8 quantisation of a bf16 [B,H,L,d] V along the key axis into the attention's tile
    layout (moc_mx_quantize_v): uint8 [B,H,Lp/64,d,80]."""
    _check_qkv(V)
    if V.dtype != torch.bfloat16:
        raise ValueError("MXFP8 quantisation takes bf16 input")
    B, H, Lq, d = V.shape
    Lp = (Lq + 63) // 64 * 64
    shape = (B, H, Lp // 64, d, VQ_ROW)
    s = lay.struct(B, H, d, V.dtype)
    n = int(L.load().moc_mx_quantize_v_bytes(ctypes.byref(s)))
    if n != math.prod(shape):
        raise L.MocError(L.MOC_EINVAL, "quantised V size does not match the tile layout")
    if out is None or tuple(out.shape) != shape:
        out = torch.empty(shape, dtype=torch.uint8, device=V.device)
    L.check(L.load().moc_mx_quantize_v(ctypes.byref(s), _ptr(V), _ptr(out), _stream(V.device)))
    return out


def attend_fwd_mxv(Qm: MxTensor, Km: MxTensor, Vq: torch.Tensor, lay: DeviceLayout, vl: Varlen,
                   scale: Optional[float] = None, ws: Optional[torch.Tensor] = None):
    """Forward with quantised scores and values (moc_attend_fwd_mxv): (O [B,H,L,d] bf16,
    lse [B,H,L])."""
    B, H, Lp, d = Qm.codes.shape
    Lq = Qm.L
    for m in (Qm, Km):
        if m.codes.shape != (B, H, Lp, d) or m.scales.shape != (B, H, Lp, d // 32):
            raise ValueError("MXFP8 operands do not match")
    if tuple(Vq.shape) != (B, H, Lp // 64, d, VQ_ROW) or Vq.dtype != torch.uint8:
        raise ValueError("quantised V does not match the MXFP8 operands")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = torch.empty((B, H, Lq, d), dtype=torch.bfloat16, device=Vq.device)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=Vq.device)
    need = vl.workspace_bytes(L.MOC_OP_FWD)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=Vq.device)
    s = lay.struct(B, H, d, torch.bfloat16)
    L.check(L.load().moc_attend_fwd_mxv(ctypes.byref(s), ctypes.byref(vl.struct), _ptr(Qm.codes),
                                        _ptr(Qm.scales), _ptr(Km.codes), _ptr(Km.scales),
                                        _ptr(Vq), float(scale), _ptr(O), _ptr(lse), _ptr(ws),
                                        ws.numel(), _stream(Vq.device)))
    return O, lse


def attend_bwd(Q, K, V, O, lse, dO, lay: DeviceLayout, vl: Varlen, scale: Optional[float] = None,
               ws: Optional[torch.Tensor] = None):
    """(dQ, dK, dV) in the input dtype."""
    _check_qkv(Q, K, V, O, dO)
    B, H, Lq, d = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dQ = torch.empty_like(Q)
    dK = torch.empty_like(K)
    dV = torch.empty_like(V)
    need = vl.workspace_bytes(L.MOC_OP_BWD)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    s = lay.struct(B, H, d, Q.dtype)
    lib = L.load()
    L.check(lib.moc_attend_bwd(ctypes.byref(s), ctypes.byref(vl.struct), _ptr(Q), _ptr(K), _ptr(V),
                               _ptr(O), _ptr(lse), _ptr(dO), float(scale), _ptr(dQ), _ptr(dK),
                               _ptr(dV), _ptr(ws), ws.numel(), _stream(Q.device)))
    return dQ, dK, dV


@dataclass
class ForwardResult:
    O: torch.Tensor
    lse: torch.Tensor
    kbar: torch.Tensor
    sel: torch.Tensor
    nsel: torch.Tensor
    varlen: Varlen


def forward(Q, K, V, lay: DeviceLayout, cfg: RouteCfg, scale: Optional[float] = None
            ) -> ForwardResult:
    """The whole layer: pool -> route -> index inversion -> attention."""
    kbar = pool_keys(K, lay)
    sel, nsel = route(Q, kbar, lay, cfg)
    vl = build_varlen(sel, nsel, lay, cfg, Q.shape[-1], Q.dtype)
    O, lse = attend_fwd(Q, K, V, lay, vl, scale)
    return ForwardResult(O, lse, kbar, sel, nsel, vl)


class MoCAttention(torch.autograd.Function):
    """Autograd wrapper: routing is a discrete choice (no gradient); gradients flow to Q, K, V
    through the attention over the selected keys and values."""

    @staticmethod
    def forward(ctx, Q, K, V, lay: DeviceLayout, cfg: RouteCfg, scale: Optional[float] = None):
        r = forward(Q, K, V, lay, cfg, scale)
        ctx.save_for_backward(Q, K, V, r.O, r.lse)
        ctx.lay, ctx.vl, ctx.scale = lay, r.varlen, scale
        return r.O

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, O, lse = ctx.saved_tensors
        dQ, dK, dV = attend_bwd(Q, K, V, O, lse, dO.contiguous(), ctx.lay, ctx.vl, ctx.scale)
        return dQ, dK, dV, None, None, None
