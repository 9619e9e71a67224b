"""ctypes view of libmoc.so (include/moc.h). Marshalling only: no arithmetic of the layer here."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_uint64, c_void_p

# The in-tree build; MOC_LIB_PATH may name another build of the same library (to compare kernel
# variants of one source tree). There is no fallback of any kind when the library is missing.
LIB_PATH = os.environ.get("MOC_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoc.so")

MOC_OK, MOC_EINVAL, MOC_ESHAPE, MOC_EDTYPE, MOC_EWORKSPACE, MOC_EUNSUPPORTED, MOC_EHIP, \
    MOC_EINTERNAL, MOC_ELAYOUT = range(9)
MOC_VARLEN_OVER_CAPACITY, MOC_VARLEN_BAD_LAYOUT = 1, 2
# bits of the layout check word
MOC_LAYOUT_BAD_START, MOC_LAYOUT_NOT_INCREASING, MOC_LAYOUT_BAD_END, MOC_LAYOUT_BAD_SHOT_ID, \
    MOC_LAYOUT_BAD_TEXT, MOC_LAYOUT_SHOT_SPLIT = 1, 2, 4, 8, 16, 32
MOC_F32, MOC_BF16 = 0, 1
MOC_OP_ROUTE, MOC_OP_VARLEN, MOC_OP_FWD, MOC_OP_BWD, MOC_OP_OUTER = range(5)
MOC_MAX_C, MOC_MAX_TOPK, MOC_MAX_DROP_IN = 1024, 32, 16
MOC_MAX_SEG, MOC_MAX_TOPM = 256, 16

# every function include/moc.h declares
EXPORTS = (
    "moc_sel_width", "moc_workspace_bytes", "moc_pool_keys", "moc_route", "moc_route_outer",
    "moc_route_masked", "moc_build_varlen", "moc_attend_fwd", "moc_attend_bwd",
    "moc_mx_quantize", "moc_attend_fwd_mx", "moc_poisson_thresholds", "moc_status_string",
    "moc_last_error", "moc_check_layout", "moc_layout_check_host", "moc_layout_status",
    "moc_route_noalloc", "moc_varlen_total", "moc_varlen_set_capacity",
    "moc_attend_workspace_bytes", "moc_varlen_status", "moc_mx_quantize_v_bytes",
    "moc_mx_quantize_v", "moc_attend_fwd_mxv",
)


class MocLayout(ctypes.Structure):
    _fields_ = [("B", c_int32), ("H", c_int32), ("L", c_int32), ("d", c_int32),
                ("dtype", c_int32), ("C", c_int32), ("chunk_offsets", c_void_p),
                ("chunk_shot", c_void_p), ("text_begin", c_int32), ("text_end", c_int32),
                ("check", c_void_p)]


class MocRouteCfg(ctypes.Structure):
    _fields_ = [("top_k", c_int32), ("causal", c_int32), ("p_max", c_float), ("lambda_", c_float),
                ("max_drop_in", c_int32), ("reserved", c_int32), ("seed", c_uint64)]


class MocVarlen(ctypes.Structure):
    _fields_ = [("S", c_int32), ("tile_rows", c_int32), ("max_rtiles", c_int32),
                ("max_atiles", c_int32), ("bucket_off", c_void_p), ("bucket_q", c_void_p),
                ("slot", c_void_p), ("rtiles", c_void_p), ("n_rtiles", c_void_p),
                ("atiles", c_void_p), ("n_atiles", c_void_p), ("scratch", c_void_p),
                ("max_ktiles", c_int32), ("n_text_split", c_int32), ("ktiles", c_void_p),
                ("n_ktiles", c_void_p), ("routed_max", c_int64), ("routed_cap", c_int64),
                ("status", c_void_p)]


class MocError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libmoc.so (built in-tree by `python sparse_chunk_routed_amd/build.py`). There is no
    fallback: a missing library is an error."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python sparse_chunk_routed_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = POINTER
    lib.moc_sel_width.argtypes = [P(MocRouteCfg), c_int32]
    lib.moc_sel_width.restype = c_int32
    lib.moc_workspace_bytes.argtypes = [P(MocLayout), P(MocRouteCfg), c_int32]
    lib.moc_workspace_bytes.restype = c_size_t
    lib.moc_pool_keys.argtypes = [P(MocLayout), c_void_p, c_void_p, c_void_p]
    lib.moc_pool_keys.restype = c_int32
    lib.moc_route.argtypes = [P(MocLayout), P(MocRouteCfg), c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_size_t, c_void_p]
    lib.moc_route.restype = c_int32
    lib.moc_route_outer.argtypes = [P(MocLayout), c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                    c_void_p]
    lib.moc_route_outer.restype = c_int32
    lib.moc_route_noalloc.argtypes = [P(MocLayout), P(MocRouteCfg), c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p]
    lib.moc_route_noalloc.restype = c_int32
    lib.moc_route_masked.argtypes = [P(MocLayout), P(MocRouteCfg), c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.moc_route_masked.restype = c_int32
    lib.moc_build_varlen.argtypes = [P(MocLayout), P(MocRouteCfg), c_void_p, c_void_p,
                                     P(MocVarlen), c_void_p, c_void_p, c_size_t, c_void_p]
    lib.moc_build_varlen.restype = c_int32
    lib.moc_attend_fwd.argtypes = [P(MocLayout), P(MocVarlen), c_void_p, c_void_p, c_void_p,
                                   c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.moc_attend_fwd.restype = c_int32
    lib.moc_attend_bwd.argtypes = [P(MocLayout), P(MocVarlen), c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_size_t, c_void_p]
    lib.moc_attend_bwd.restype = c_int32
    lib.moc_mx_quantize.argtypes = [P(MocLayout), c_void_p, c_void_p, c_void_p, c_void_p]
    lib.moc_mx_quantize.restype = c_int32
    lib.moc_attend_fwd_mx.argtypes = [P(MocLayout), P(MocVarlen), c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_float, c_void_p, c_void_p, c_void_p,
                                      c_size_t, c_void_p]
    lib.moc_attend_fwd_mx.restype = c_int32
    lib.moc_mx_quantize_v_bytes.argtypes = [P(MocLayout)]
    lib.moc_mx_quantize_v_bytes.restype = c_size_t
    lib.moc_mx_quantize_v.argtypes = [P(MocLayout), c_void_p, c_void_p, c_void_p]
    lib.moc_mx_quantize_v.restype = c_int32
    lib.moc_attend_fwd_mxv.argtypes = [P(MocLayout), P(MocVarlen), c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_float, c_void_p, c_void_p, c_void_p,
                                       c_size_t, c_void_p]
    lib.moc_attend_fwd_mxv.restype = c_int32
    lib.moc_poisson_thresholds.argtypes = [c_float, c_int32, P(c_uint64)]
    lib.moc_poisson_thresholds.restype = c_int32
    lib.moc_check_layout.argtypes = [P(MocLayout), c_void_p]
    lib.moc_check_layout.restype = c_int32
    lib.moc_layout_check_host.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32]
    lib.moc_layout_check_host.restype = ctypes.c_uint32
    lib.moc_layout_status.argtypes = [ctypes.c_uint32]
    lib.moc_layout_status.restype = c_int32
    lib.moc_varlen_total.argtypes = [P(MocLayout), P(MocVarlen), P(c_int64), c_void_p]
    lib.moc_varlen_total.restype = c_int32
    lib.moc_varlen_set_capacity.argtypes = [P(MocVarlen), c_int64]
    lib.moc_varlen_set_capacity.restype = c_int32
    lib.moc_attend_workspace_bytes.argtypes = [P(MocLayout), P(MocVarlen), c_int32]
    lib.moc_attend_workspace_bytes.restype = c_size_t
    lib.moc_varlen_status.argtypes = [P(MocVarlen), c_void_p]
    lib.moc_varlen_status.restype = c_int32
    lib.moc_status_string.argtypes = [c_int32]
    lib.moc_status_string.restype = c_char_p
    lib.moc_last_error.argtypes = []
    lib.moc_last_error.restype = c_char_p
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != MOC_OK:
        lib = load()
        raise MocError(status, lib.moc_last_error().decode(errors="replace"))
