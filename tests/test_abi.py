"""C-ABI checks that need no GPU: the library loads, exports every function include/moc.h
declares, validates arguments before enqueueing anything, sizes workspaces monotonically, and
computes the drop-in thresholds the oracle computes."""
import ctypes
import os
import re

import numpy as np
import pytest

import moc_inputs as mi
from oracle import rng as orng

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from sparse_chunk_routed_amd import _lib
    _lib.load()
    return _lib


def _decls():
    src = open(os.path.join(ROOT, "include", "moc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moc_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    lib = L.load()
    decls = _decls()
    assert set(decls) == set(L.EXPORTS), decls
    for name in decls:
        assert hasattr(lib, name), name
    # and the symbols are plain C (unmangled) in the ELF dynamic table
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True).stdout
    for name in decls:
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def _layout(L, B=1, H=2, d=64, dtype=0, w=None, **over):
    w = w or mi.tiny()
    lay = w.layout
    s = L.MocLayout(B, H, lay.L, d, dtype, lay.C, 0x1000, 0x2000, lay.text_begin, lay.text_end)
    for k, v in over.items():
        setattr(s, k, v)
    return s


def _cfg(L, **over):
    c = L.MocRouteCfg(2, 1, 0.0, 0.0, 8, 0, 0)
    for k, v in over.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("over,status", [
    ({"d": 96}, 2), ({"dtype": 7}, 3), ({"C": 0}, 2), ({"C": 5000}, 2), ({"B": 0}, 2),
    ({"chunk_offsets": None}, 1), ({"text_end": 10 ** 7}, 1), ({"text_begin": 5, "text_end": 4}, 1),
])
def test_layout_validation(L, over, status):
    lib = L.load()
    s = _layout(L, **over)
    kbar = ctypes.c_void_p(0x3000)
    assert lib.moc_pool_keys(ctypes.byref(s), ctypes.c_void_p(0x4000), kbar, None) == status
    assert lib.moc_last_error().decode().startswith(lib.moc_status_string(status).decode())


@pytest.mark.parametrize("over,status", [
    ({"top_k": -1}, 1), ({"causal": 2}, 1), ({"p_max": 1.5}, 1), ({"lambda_": -1.0}, 1),
    ({"max_drop_in": 17}, 2), ({"top_k": 40}, 0),
])
def test_route_cfg_validation(L, over, status):
    lib = L.load()
    lay = _layout(L)
    cfg = _cfg(L, **over)
    if status == 0:
        # top_k beyond C means "all": valid, and S = C
        assert lib.moc_sel_width(ctypes.byref(cfg), lay.C) == lay.C
        return
    r = lib.moc_route(ctypes.byref(lay), ctypes.byref(cfg), ctypes.c_void_p(1), ctypes.c_void_p(2),
                      ctypes.c_void_p(3), ctypes.c_void_p(4), None, 0, None)
    assert r == status


def test_topk_limit(L):
    lib = L.load()
    lay = mi.build_layout(0, [40], 8)
    s = L.MocLayout(1, 1, lay.L, 64, 0, lay.C, 1, 1, 0, 0)
    cfg = _cfg(L, top_k=33)
    r = lib.moc_route(ctypes.byref(s), ctypes.byref(cfg), ctypes.c_void_p(1), ctypes.c_void_p(2),
                      ctypes.c_void_p(3), ctypes.c_void_p(4), None, 0, None)
    assert r == 2


def test_null_and_alias_rejected(L):
    lib = L.load()
    lay = _layout(L)
    assert lib.moc_pool_keys(ctypes.byref(lay), None, ctypes.c_void_p(8), None) == 1
    assert lib.moc_pool_keys(ctypes.byref(lay), ctypes.c_void_p(8), ctypes.c_void_p(8), None) == 1
    cfg = _cfg(L)
    vl = L.MocVarlen()
    pc = ctypes.c_void_p(16)
    # workspace too small
    assert lib.moc_build_varlen(ctypes.byref(lay), ctypes.byref(cfg), ctypes.c_void_p(1),
                                ctypes.c_void_p(2), ctypes.byref(vl), pc, ctypes.c_void_p(64), 10,
                                None) == 4
    # attention with an unfilled varlen struct
    assert lib.moc_attend_fwd(ctypes.byref(lay), ctypes.byref(vl), ctypes.c_void_p(1),
                              ctypes.c_void_p(2), ctypes.c_void_p(3), ctypes.c_float(0.125),
                              ctypes.c_void_p(4), ctypes.c_void_p(5), ctypes.c_void_p(6), 1 << 30,
                              None) == 1


def test_workspace_monotone(L):
    lib = L.load()
    prev = None
    for frames in (1, 2, 4, 8):
        lay = mi.build_layout(16, [frames] * 3, 64)
        s = L.MocLayout(1, 2, lay.L, 64, 1, lay.C, 1, 1, lay.text_begin, lay.text_end)
        sizes = []
        for k in (1, 2, 4):
            for lam in (0.0, 1.0):
                cfg = _cfg(L, top_k=k, lambda_=lam)
                sizes.append(tuple(lib.moc_workspace_bytes(ctypes.byref(s), ctypes.byref(cfg), op)
                                   for op in (1, 2)))
        cur = sizes[0]
        if prev is not None:
            assert cur[0] >= prev[0] and cur[1] >= prev[1]
        prev = cur
    lay = mi.tiny().layout
    s = L.MocLayout(1, 2, lay.L, 64, 0, lay.C, 1, 1, lay.text_begin, lay.text_end)
    w = [lib.moc_workspace_bytes(ctypes.byref(s), ctypes.byref(_cfg(L, top_k=k)), 2)
         for k in range(0, 6)]
    assert all(b >= a for a, b in zip(w, w[1:]))


def test_sel_width(L):
    lib = L.load()
    assert lib.moc_sel_width(ctypes.byref(_cfg(L, top_k=2)), 17) == 2
    assert lib.moc_sel_width(ctypes.byref(_cfg(L, top_k=2, lambda_=1.0, max_drop_in=8)), 17) == 10
    assert lib.moc_sel_width(ctypes.byref(_cfg(L, top_k=50)), 17) == 17
    assert lib.moc_sel_width(ctypes.byref(_cfg(L, top_k=0)), 17) == 0


@pytest.mark.parametrize("lam", [0.25, 1.0, 3.0])
def test_poisson_thresholds_match_oracle(L, lam):
    lib = L.load()
    arr = (ctypes.c_uint64 * 16)()
    assert lib.moc_poisson_thresholds(ctypes.c_float(lam), 16, arr) == 0
    ref = orng.poisson_thresholds(float(np.float32(lam)), 16)
    assert list(arr) == ref


def test_python_layout_validation():
    from sparse_chunk_routed_amd.api import validate_layout
    lay = mi.tiny().layout
    validate_layout(np.asarray(lay.chunk_offsets), np.asarray(lay.chunk_shot), lay.text_begin,
                    lay.text_end)
    with pytest.raises(ValueError):
        validate_layout(np.array([0, 3, 2]), np.array([0, 1]), 0, 0)
    with pytest.raises(ValueError):
        validate_layout(np.array([0, 3, 6, 9]), np.array([0, 1, 0]), 0, 0)
    with pytest.raises(ValueError):
        validate_layout(np.array([0, 3, 6]), np.array([-1, 0]), 0, 2)


@pytest.mark.parametrize("nseg,M,causal,status", [
    (0, 1, 1, 2),          # no segment
    (300, 1, 1, 2),        # beyond MOC_MAX_SEG (and C)
    (5, -1, 1, 1),         # negative M
    (5, 1, 2, 1),          # bad causal flag
    (17, 17, 1, 2),        # min(M, nseg) beyond MOC_MAX_TOPM
])
def test_route_outer_validation(L, nseg, M, causal, status):
    lib = L.load()
    lay = _layout(L)
    p = ctypes.c_void_p
    r = lib.moc_route_outer(ctypes.byref(lay), p(1), nseg, M, causal, p(2), p(3), p(4), p(5),
                            p(6), p(7), 1 << 30, None)
    assert r == status, lib.moc_last_error()


def test_route_outer_and_masked_reject_null_and_small_workspace(L):
    lib = L.load()
    lay = _layout(L)
    p = ctypes.c_void_p
    need = lib.moc_workspace_bytes(ctypes.byref(lay), ctypes.byref(_cfg(L)), L.MOC_OP_OUTER)
    assert need > 0
    assert lib.moc_route_outer(ctypes.byref(lay), None, 5, 1, 1, p(2), p(3), p(4), p(5), p(6),
                               p(7), need, None) == 1
    assert lib.moc_route_outer(ctypes.byref(lay), p(1), 5, 1, 1, p(2), p(3), p(4), p(5), p(6),
                               p(7), need - 1, None) == 4
    cfg = _cfg(L)
    assert lib.moc_route_masked(ctypes.byref(lay), ctypes.byref(cfg), p(1), p(2), None, p(3),
                                p(4), None, 0, None) == 1
    assert lib.moc_route_masked(ctypes.byref(lay), ctypes.byref(_cfg(L, top_k=-1)), p(1), p(2),
                                p(9), p(3), p(4), None, 0, None) == 1


def test_device_segments_validation():
    """Segments are checked on the host copy against the layout before any device call."""
    import moc_inputs as mi
    import sparse_chunk_routed_amd as moc
    lay = moc.DeviceLayout.from_layout(mi.build_layout(16, [3, 3, 3, 3], 12), "cpu")
    s = moc.DeviceSegments([0, 1, 4, 6, 10, 13], lay)
    assert s.nseg == 5 and s.host == [0, 1, 4, 6, 10, 13]
    for bad in ([0, 2, 13], [0, 1, 1, 13], [0, 1, 12], [1, 13], [0]):
        with pytest.raises(ValueError):
            moc.DeviceSegments(bad, lay)


def test_mx_entry_points_reject_bad_arguments(L):
    """Host-side validation of the quantised-scores entry points (nothing is launched)."""
    lib = L.load()
    p = ctypes.c_void_p
    f32 = _layout(L, dtype=0)
    bf = _layout(L, dtype=1)
    assert lib.moc_mx_quantize(ctypes.byref(f32), p(1), p(2), p(3), None) == 3   # dtype
    assert lib.moc_mx_quantize(ctypes.byref(bf), None, p(2), p(3), None) == 1    # NULL
    assert lib.moc_mx_quantize(ctypes.byref(bf), p(1), p(2), p(2), None) == 1    # alias
    assert lib.moc_mx_quantize(ctypes.byref(_layout(L, dtype=1, d=96)), p(1), p(2), p(3),
                               None) == 2                                        # d
    vl = L.MocVarlen()
    assert lib.moc_attend_fwd_mx(ctypes.byref(bf), ctypes.byref(vl), p(1), p(2), p(3), p(4),
                                 p(5), ctypes.c_float(0.125), p(6), p(7), p(8), 1 << 30,
                                 None) == 1                                      # unfilled varlen
    assert lib.moc_attend_fwd_mx(ctypes.byref(bf), None, p(1), p(2), p(3), p(4), p(5),
                                 ctypes.c_float(0.125), p(6), p(7), p(8), 1 << 30, None) == 1


def test_bench_probe_library_is_separate_and_rejects_bad_arguments(L):
    """The benchmark's MFMA probe lives in its own library, not in libmoc."""
    path = os.path.join(ROOT, "sparse_chunk_routed_amd", "libmoc_bench_probe.so")
    probe = ctypes.CDLL(path)
    f = probe.moc_bench_probe_mfma
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    p = ctypes.c_void_p
    assert f(2, 1, 1, p(8), None) == 1
    assert f(0, 0, 1, p(8), None) == 1
    assert f(0, 1, 0, p(8), None) == 1
    assert f(1, 1, 1, None, None) == 1
    assert not hasattr(L.load(), "moc_bench_probe_mfma")
    assert not hasattr(L.load(), "moc_probe_mfma")


# ---------------------------------------------------------------------------------------------
# Layout content check (moc_layout.check): the host build of the same check function the device
# kernel runs.
# ---------------------------------------------------------------------------------------------

def _host_bits(L, lay):
    from sparse_chunk_routed_amd.api import layout_check_host
    return layout_check_host(lay.chunk_offsets, lay.chunk_shot, lay.text_begin, lay.text_end)


def test_layout_check_host_accepts_valid_layouts(L):
    for name in ("tiny", "short", "headline", "single_shot_c64", "headline_outer"):
        assert _host_bits(L, mi.WORKLOADS[name]().layout) == 0, name
    for seed in range(50):
        rng = np.random.default_rng(seed)
        lay = mi.make_random_layout(rng, max_shots=6, max_frames=4, max_chunk=30,
                                    frame_is_shot=bool(seed % 4 == 0))
        assert _host_bits(L, lay) == 0, seed


@pytest.mark.parametrize("case,bit", [
    ("start", 1), ("order", 2), ("end", 4), ("shot_id", 8), ("text_tag", 16),
    ("straddle", 16), ("text_outside", 16), ("shot_split", 32),
])
def test_layout_check_host_flags_each_violation(L, case, bit):
    from sparse_chunk_routed_amd.api import layout_check_host
    off = np.array([0, 4, 10, 13, 20, 26], dtype=np.int32)  # text [0,4), shots 0,0,1,1
    shot = np.array([-1, 0, 0, 1, 1], dtype=np.int32)
    tb, te, Lt = 0, 4, 26
    if case == "start":
        off = off + 1
        Lt = int(off[-1])
    elif case == "order":
        off[3] = 10  # chunk 2 becomes empty
    elif case == "end":
        Lt = 30
    elif case == "shot_id":
        shot[3] = -2
    elif case == "text_tag":
        shot[0] = 5
    elif case == "straddle":
        te = 6
    elif case == "text_outside":
        shot[4] = -1
    elif case == "shot_split":
        shot = np.array([-1, 0, 1, 0, 2], dtype=np.int32)
    bits = int(L.load().moc_layout_check_host(off.ctypes.data, shot.ctypes.data, 5, Lt, tb, te))
    assert bits & bit, (case, bits)
    if case not in ("start",):  # shifting every offset also breaks the text alignment
        assert bits == bit, (case, bits)
    st = L.load().moc_layout_status(bits)
    assert st == L.MOC_ELAYOUT
    assert "layout check word" in L.load().moc_last_error().decode()
    assert L.load().moc_layout_status(0) == 0


def test_layout_check_host_agrees_with_the_validators(L):
    """Random single mutations of random layouts: the library's check flags a layout exactly
    when the Python binding's validator and the oracle's derive() reject it."""
    from oracle import moc_oracle as mo
    from sparse_chunk_routed_amd.api import validate_layout
    rng = np.random.default_rng(123)
    n_bad = 0
    for it in range(3000):
        lay = mi.make_random_layout(rng, max_shots=4, max_frames=3, max_chunk=8,
                                    frame_is_shot=bool(rng.integers(0, 2)))
        off = np.array(lay.chunk_offsets, dtype=np.int64)
        shot = np.array(lay.chunk_shot, dtype=np.int64)
        tb, te = lay.text_begin, lay.text_end
        kind = int(rng.integers(0, 5))
        C = len(shot)
        if kind == 0 and C > 1:
            i = int(rng.integers(1, C))
            off[i] = int(rng.integers(off[i - 1] - 1, off[i + 1] + 2))
        elif kind == 1:
            shot[int(rng.integers(0, C))] = int(rng.integers(-2, 5))
        elif kind == 2:
            tb = int(rng.integers(0, off[-1] + 1))
            te = int(rng.integers(tb, off[-1] + 1))
        elif kind == 3 and C > 1:
            i, j = rng.choice(C, 2, replace=False)
            shot[i], shot[j] = shot[j], shot[i]
        o32, s32 = off.astype(np.int32), shot.astype(np.int32)
        bits = int(L.load().moc_layout_check_host(o32.ctypes.data, s32.ctypes.data, C,
                                                   int(off[-1]), tb, te))
        try:
            validate_layout(off, shot, tb, te)
            py_ok = True
        except ValueError:
            py_ok = False
        try:
            mo.derive(mi.Layout(off, shot, tb, te))
            or_ok = True
        except ValueError:
            or_ok = False
        assert py_ok == or_ok == (bits == 0), (it, kind, off.tolist(), shot.tolist(), tb, te,
                                               bits, py_ok, or_ok)
        n_bad += bits != 0
    assert n_bad > 500


def test_route_noalloc_rejects_requests_beyond_its_static_buffer(L):
    """moc_route_noalloc keeps the kbar split (B*H*C*d*6 bytes for bf16) in a 16 MiB static
    buffer: a larger request is refused on the host before anything is enqueued."""
    lib = L.load()
    lay = mi.build_layout(0, [1024], 2)  # 1,024 single-frame chunks, L = 2,048
    ok = L.MocLayout(1, 12, lay.L, 128, 1, lay.C, 1, 1, 0, 0)   # 12*1024*128*6 = 9.4 MiB
    big = L.MocLayout(1, 24, lay.L, 128, 1, lay.C, 1, 1, 0, 0)  # 18.9 MiB
    cfg = _cfg(L, top_k=2)
    p = ctypes.c_void_p
    assert lib.moc_route_noalloc(ctypes.byref(big), ctypes.byref(cfg), p(1), p(2), p(3), p(4),
                                 None) == L.MOC_ESHAPE
    assert "16777216-byte static buffer" in lib.moc_last_error().decode()
    assert lib.moc_workspace_bytes(ctypes.byref(ok), ctypes.byref(cfg), L.MOC_OP_ROUTE) <= 16 << 20
    # the usual argument checks still run first
    assert lib.moc_route_noalloc(None, ctypes.byref(cfg), p(1), p(2), p(3), p(4), None) == 1


def test_varlen_set_capacity_bounds(L):
    """The routed-row capacity of the attention workspaces lies in [0, routed_max]; a struct that
    moc_build_varlen did not fill is refused."""
    lib = L.load()
    vl = L.MocVarlen()
    assert lib.moc_varlen_set_capacity(ctypes.byref(vl), 10) == L.MOC_EINVAL  # not filled
    vl.status = 0x1000
    vl.routed_max = 1000
    vl.routed_cap = 1000
    assert lib.moc_varlen_set_capacity(ctypes.byref(vl), -1) == L.MOC_EINVAL
    assert lib.moc_varlen_set_capacity(ctypes.byref(vl), 1001) == L.MOC_EINVAL
    assert vl.routed_cap == 1000
    assert lib.moc_varlen_set_capacity(ctypes.byref(vl), 0) == 0 and vl.routed_cap == 0
    assert lib.moc_varlen_set_capacity(ctypes.byref(vl), 1000) == 0 and vl.routed_cap == 1000
    assert lib.moc_varlen_set_capacity(None, 5) == L.MOC_EINVAL
