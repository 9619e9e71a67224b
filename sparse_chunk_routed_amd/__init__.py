"""Mixture-of-Contexts (MoC) attention layer for AMD MI355X (gfx950).

The layer's steps run in hand-written HIP kernels behind the C ABI of libmoc.so
(include/moc.h); this package loads that library and exposes the same entry points for torch
tensors. Importing it fails if libmoc.so has not been built.
"""
from . import _lib
from ._lib import MocError, load
from .api import (DeviceLayout, DeviceSegments, ForwardResult, MoCAttention, MxTensor,
                  OuterRouting, RouteCfg, Varlen, attend_bwd, attend_fwd, attend_fwd_mx,
                  attend_fwd_mxv, build_varlen, forward, mx_quantize, mx_quantize_v, pool_keys,
                  route, route_outer,
                  layout_check_host, sel_width, validate_layout, workspace_bytes)

load()

__all__ = ["DeviceLayout", "DeviceSegments", "ForwardResult", "MoCAttention", "MocError",
           "MxTensor", "OuterRouting", "RouteCfg", "Varlen", "attend_bwd", "attend_fwd",
           "attend_fwd_mx", "attend_fwd_mxv", "build_varlen", "forward", "mx_quantize",
           "mx_quantize_v", "pool_keys", "route",
           "route_outer", "layout_check_host", "sel_width", "validate_layout", "workspace_bytes"]
