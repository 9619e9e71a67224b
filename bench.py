"""Benchmark of the MoC attention layer on one MI355X.

One step = one pass of the whole layer (pool -> route -> index inversion -> attention forward;
plus the backward for --workload train) over one batch of seeded synthetic input already
resident in HBM. Prints ONE JSON line.

value = effective TFLOP/s on attended pairs over the whole layer: 4*d FLOPs per attended
(query, key) pair (the dense-attention convention of the MoC summary, Eq. 5), pairs counted
exactly by the index inversion, divided by the layer time.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoC layer ms + effective TFLOP/s on attended pairs at ~175k tokens, 1 MI355X"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}  # MI355X dense MFMA (bf16), fp32
# quantised scores: per attended pair 2d FLOPs of S on fp8 (2 x the bf16 rate) and 2d of P.V
# on bf16, so the time-weighted dense peak of the pair is 4 / (2 / 5033.2 + 2 / 2516.6)
PEAK_MX_TFLOPS = 4.0 / (2.0 / (2 * 2516.6) + 2.0 / 2516.6)
PEAK_FP8_TFLOPS = 2 * 2516.6  # quantised scores and values: both products on fp8
PEAK_HBM_GBS = 8000.0


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="headline",
                    choices=["headline", "mid", "short", "tiny", "train", "headline_uniform",
                             "single_shot_c64", "single_shot_c128", "single_shot_c256",
                             "single_shot_c512", "single_shot_c1024", "headline_outer",
                             "headline_mx", "headline_mxv", "headline_h3"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=768,
                    help="query rows of the oracle attention sample (spread over the heads)")
    ap.add_argument("--sweep", default="",
                    help="comma-separated shot counts: instead of the one-line benchmark, time "
                         "the MoC layer on n shots of 21,840 tokens (+512 text) against dense "
                         "attention over the same tokens, one JSON line per n")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates the HBM "
                         "byte counters of a profiler against a known traffic)")
    return ap.parse_args(argv)


TRAFFIC_SOURCES = ["sparse_chunk_routed_amd/csrc/attn_fwd.hip",
                   "sparse_chunk_routed_amd/csrc/attn_fwd_lds.h",
                   "sparse_chunk_routed_amd/csrc/attn_common.h",
                   "sparse_chunk_routed_amd/csrc/moc_common.h"]


def recorded_traffic(workload: str):
    """HBM bytes per attention-forward call from the committed rocprofv3 counter summary of
    this workload (profiles/attention_fwd_<workload>_traffic.txt), or None when there is none
    or the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"attention_fwd_{workload}_traffic.txt")
    if not workload or not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            rec[k] = v
    h = hashlib.sha256()
    for src in TRAFFIC_SOURCES:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if h.hexdigest() != rec.get("kernel_sources_sha256"):
        return None
    return int(rec["fetch_bytes_per_launch"]) + int(rec["write_bytes_per_launch"])


def _probe_lib():
    """The benchmark's helper library (register-only MFMA loops, built next to libmoc.so by
    sparse_chunk_routed_amd/build.py); not part of the layer's library."""
    import ctypes
    path = os.path.join(ROOT, "sparse_chunk_routed_amd", "libmoc_bench_probe.so")
    lib = ctypes.CDLL(path)
    lib.moc_bench_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.moc_bench_probe_mfma.restype = ctypes.c_int
    return lib


def measured_peaks(dev) -> dict:
    """Ceilings re-measured on this GPU next to the published ones: a plain device copy (HBM
    GB/s, read + write) and register-only MFMA loops (moc_bench_probe_mfma: bf16, and fp8 with
    block scales), each the best of three timed launches after a warm-up."""
    import torch
    probe = _probe_lib()

    def probe_mfma(fp8, blocks, iters, sink):
        st = torch.cuda.current_stream(dev).cuda_stream
        rc = probe.moc_bench_probe_mfma(int(fp8), blocks, iters, sink.data_ptr(), st)
        if rc != 0:
            raise RuntimeError(f"moc_bench_probe_mfma returned {rc}")

    def best(fn, reps=3):
        fn()
        out = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            out.append(a.elapsed_time(b) * 1e-3)
        return min(out)

    n = 1 << 31
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    t_copy = best(lambda: dst.copy_(src))
    del src, dst
    blocks, iters = 1024, 4096
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    waves_mfma = blocks * 4 * iters * 8
    t_bf16 = best(lambda: probe_mfma(False, blocks, iters, sink))
    t_fp8 = best(lambda: probe_mfma(True, blocks, iters, sink))
    return {"hbm_copy_gbs": 2 * n / t_copy / 1e9,
            "mfma_bf16_tflops": waves_mfma * 2 * 32 * 32 * 16 / t_bf16 / 1e12,
            "mfma_fp8_tflops": waves_mfma * 2 * 32 * 32 * 64 / t_fp8 / 1e12,
            "how": "device copy of 2 GiB; register-only MFMA loops, 4,096 waves x 8 chains"}


def copy_calibration() -> int:
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 3}), flush=True)
    return 0


def cpu_baseline(w, Q, K, V, rows_n: int):
    """The oracle timed on a bounded sample of the same workload: pooling and routing in full
    (every head), attention on a seeded sample of query rows spread over the heads, extrapolated
    linearly to every row."""
    import numpy as np
    from oracle import moc_oracle as mo
    from threadpoolctl import threadpool_limits
    affinity = len(os.sched_getaffinity(0))  # the host cores this process may run on
    # the oracle's BLAS gets all of them, within the OpenMP thread budget when one is set
    threads = min(affinity, int(os.environ.get("OMP_NUM_THREADS", affinity) or affinity))
    limit = threadpool_limits(limits=threads)
    t0 = time.perf_counter()
    kb = mo.pool_keys(K, w.layout)
    t_pool = time.perf_counter() - t0
    t0 = time.perf_counter()
    cmask = None
    if w.segments is not None:
        cmask = mo.route_outer(Q, K, w.layout, w.segments, w.outer_M, w.causal).cand_mask
    r = mo.route(Q, kb, w.layout, w.top_k, w.causal, cand_mask=cmask)
    t_route = time.perf_counter() - t0
    rng = np.random.default_rng(w.seed)
    n = min(rows_n, w.B * w.H * w.L)
    flat = np.sort(rng.choice(w.B * w.H * w.L, size=n, replace=False))
    rows = [(int(i // (w.H * w.L)), int(i // w.L % w.H), int(i % w.L)) for i in flat]
    t0 = time.perf_counter()
    att = mo.attend_mxv if w.mx_values else mo.attend_mx if w.mx_scores else mo.attend
    att(Q, K, V, w.layout, r.sel, rows=rows)
    t_att = time.perf_counter() - t0
    measured = t_pool + t_route + t_att
    full = t_pool + t_route + t_att * (w.B * w.H * w.L / len(rows))
    pairs = int(mo.pair_counts(w.layout, r.sel).sum())
    flops = 4 * w.d * pairs
    limit.unregister()
    return {
        "value": flops / full / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "affinity_cores": affinity,
        "sample": (f"fp64 numpy oracle: pool and route on all {w.B * w.H} heads, attention on "
                   f"{len(rows)} seeded query rows across the heads; measured {measured:.1f} s "
                   f"(pool {t_pool:.1f}, route {t_route:.1f}, attention {t_att:.1f}), "
                   f"extrapolated linearly to all {w.B * w.H * w.L} rows = {full:.1f} s"),
        "measured_s": measured, "extrapolated_full_layer_s": full,
    }


def sweep(a) -> int:
    """MoC layer vs dense attention over the same tokens, for several shot counts."""
    import torch

    import moc_inputs as mi
    import sparse_chunk_routed_amd as moc

    dev = torch.device("cuda:0")

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    for n in [int(x) for x in a.sweep.split(",") if x]:
        w = mi.shots(a.seed, n_shots=n)
        wd = mi.dense(a.seed, n_shots=n)
        print(f"[bench] sweep: {n} shots, L={w.L}", file=sys.stderr, flush=True)
        Qd, Kd, Vd = (x.to(dev) for x in mi.make_qkv(w))
        lay = moc.DeviceLayout.from_layout(w.layout, dev)
        cfg = moc.RouteCfg(w.top_k, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed)
        ws = torch.empty(moc.workspace_bytes(lay, w.B, w.H, w.d, Qd.dtype, cfg, 2),
                         dtype=torch.uint8, device=dev)
        box = {}

        def layer():
            kbar = moc.pool_keys(Kd, lay)
            sel, nsel = moc.route(Qd, kbar, lay, cfg)
            box["vl"] = moc.build_varlen(sel, nsel, lay, cfg, w.d, Qd.dtype)
            moc.attend_fwd(Qd, Kd, Vd, lay, box["vl"], ws=ws)

        moc_ms = timed(layer, a.steps, a.warmup)
        pairs = int(box["vl"].pair_count.sum().item())
        del ws, box
        lay_d = moc.DeviceLayout.from_layout(wd.layout, dev)
        cfg_d = moc.RouteCfg(0, True, 0.0, 0.0, 8, wd.seed)
        kbar = moc.pool_keys(Kd, lay_d)
        sel, nsel = moc.route(Qd, kbar, lay_d, cfg_d)
        vl_d = moc.build_varlen(sel, nsel, lay_d, cfg_d, wd.d, Qd.dtype)
        dpairs = int(vl_d.pair_count.sum().item())
        assert dpairs == wd.B * wd.H * wd.L * wd.L
        ws_d = torch.empty(moc.workspace_bytes(lay_d, wd.B, wd.H, wd.d, Qd.dtype, cfg_d, 2),
                           dtype=torch.uint8, device=dev)
        dense_ms = timed(lambda: moc.attend_fwd(Qd, Kd, Vd, lay_d, vl_d, ws=ws_d),
                         max(1, a.steps // 2), 1)
        print(json.dumps({
            "sweep": "shots", "n_shots": n, "L": w.L, "B": w.B, "H": w.H, "d": w.d,
            "moc_layer_ms": moc_ms, "dense_attention_ms": dense_ms,
            "speedup": dense_ms / moc_ms, "pairs": pairs, "dense_pairs": dpairs,
            "pruned_fraction": 1.0 - pairs / dpairs,
            "moc_tflops": 4 * w.d * pairs / (moc_ms * 1e-3) / 1e12,
            "dense_tflops": 4 * wd.d * dpairs / (dense_ms * 1e-3) / 1e12}), flush=True)
        del Qd, Kd, Vd, ws_d, vl_d, sel, nsel, kbar
        torch.cuda.empty_cache()
    return 0


def main(argv=None) -> int:
    a = parse(argv)
    if a.copy_calibration:
        return copy_calibration()
    if a.sweep:
        if a.gpus != 1:
            print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
            return 2
        return sweep(a)
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        return 2
    import torch

    import moc_inputs as mi
    import sparse_chunk_routed_amd as moc

    dev = torch.device("cuda:0")
    w = mi.WORKLOADS[a.workload](a.seed)
    with_bwd = a.workload == "train"
    print(f"[bench] workload {w.name}: {w.description}; B={w.B} H={w.H} L={w.L} d={w.d} "
          f"C={w.C} k={w.top_k}", file=sys.stderr, flush=True)
    tensors = mi.make_qkv(w, with_dout=with_bwd)
    Q, K, V = tensors[:3]
    Qd, Kd, Vd = (x.to(dev) for x in (Q, K, V))
    dOd = tensors[3].to(dev) if with_bwd else None
    lay = moc.DeviceLayout.from_layout(w.layout, dev)
    cfg = moc.RouteCfg(w.top_k, w.causal, w.p_max, w.lam, w.max_drop_in, w.seed)
    # the attention workspaces are sized for the routing's real total of routed rows (read once,
    # in an untimed first pass; the inputs are the same every step), not for the static bound
    # B*H*L*S
    cap = {"rows": None}
    fwd_ws = bwd_ws = None

    outer = w.segments is not None
    segs = moc.DeviceSegments(w.segments, lay) if outer else None
    mx = w.mx_scores
    mxv = w.mx_values
    qm = km = vq = None
    names = (["pool"] + (["route_outer"] if outer else []) + ["route", "varlen"]
             + (["mx_quantize"] if mx else []) + ["attend_fwd"]
             + (["attend_bwd"] if with_bwd else []))

    def step(ev=None):
        nonlocal qm, km, vq
        i = 0

        def mark():
            nonlocal i
            if ev is not None:
                ev[i].record()
            i += 1
        mark()
        kbar = moc.pool_keys(Kd, lay)
        mark()
        cand_mask = None
        if outer:
            cand_mask = moc.route_outer(Qd, Kd, lay, segs, w.outer_M, w.causal).cand_mask
            mark()
        sel, nsel = moc.route(Qd, kbar, lay, cfg, cand_mask=cand_mask)
        mark()
        vl = moc.build_varlen(sel, nsel, lay, cfg, w.d, Qd.dtype)
        if cap["rows"] is not None:
            vl.set_capacity(cap["rows"])
        mark()
        if mx:
            qm = moc.mx_quantize(Qd, lay, out=qm)
            km = moc.mx_quantize(Kd, lay, out=km)
            if mxv:
                vq = moc.mx_quantize_v(Vd, lay, out=vq)
            mark()
            if mxv:
                O, lse = moc.attend_fwd_mxv(qm, km, vq, lay, vl, ws=fwd_ws)
            else:
                O, lse = moc.attend_fwd_mx(qm, km, Vd, lay, vl, ws=fwd_ws)
        else:
            O, lse = moc.attend_fwd(Qd, Kd, Vd, lay, vl, ws=fwd_ws)
        mark()
        if with_bwd:
            moc.attend_bwd(Qd, Kd, Vd, O, lse, dOd, lay, vl, ws=bwd_ws)
            mark()
        return vl

    # one untimed pass at the default capacity gives the routing's total and the default sizes
    vl0 = step()
    ws_default = {"fwd": vl0.workspace_bytes(2), "bwd": vl0.workspace_bytes(3)}
    cap["rows"] = vl0.total()
    vl0.set_capacity(cap["rows"])
    ws_used = {"fwd": vl0.workspace_bytes(2), "bwd": vl0.workspace_bytes(3)}
    # the forward's workspace is dead once it returns (the backward reads O and lse, not the
    # partial rows), so a step's forward and backward share one buffer of the larger size
    fwd_ws = torch.empty(max(ws_used["fwd"], ws_used["bwd"] if with_bwd else 0),
                         dtype=torch.uint8, device=dev)
    bwd_ws = fwd_ws if with_bwd else None
    del vl0
    torch.cuda.empty_cache()

    for _ in range(a.warmup):
        vl = step()
    torch.cuda.synchronize()
    if a.warmup:
        vl.check_status()  # every routed row fitted the capacity
    print(f"[bench] warmup done ({a.warmup} steps)", file=sys.stderr, flush=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(a.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(a.steps):
        vl = step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    vl.check_status()  # the timed steps' routed rows fitted the capacity too
    total_ms = t_start.elapsed_time(t_end)
    ms = total_ms / a.steps
    step_ms = sorted(e[0].elapsed_time(e[-1]) for e in evs)
    stage = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / a.steps
             for j, n in enumerate(names)}
    pairs = int(vl.pair_count.sum().item())
    fwd_flops = 4 * w.d * pairs
    bwd_flops = 10 * w.d * pairs if with_bwd else 0
    flops = fwd_flops + bwd_flops
    s_in = 2 if w.dtype == "bf16" else 4
    BHLd = w.B * w.H * w.L * w.d
    S = moc.sel_width(cfg, w.C)
    pool_bytes = BHLd * s_in + w.B * w.H * w.C * w.d * 4
    route_bytes = BHLd * s_in + w.B * w.H * w.C * w.d * 4 + w.B * w.H * w.L * (S + 1) * 4
    # the index inversion (the gather that lets a query tile read a chunk's K/V once): sel and
    # nsel read by the count pass and again by the scatter pass, one bucket_q and one slot int32
    # written per routed row
    gather_bytes = 2 * w.B * w.H * w.L * (S + 1) * 4 + 2 * cap["rows"] * 4
    peak = PEAK_FP8_TFLOPS if mxv else PEAK_MX_TFLOPS if mx else PEAK_TFLOPS[w.dtype]
    att_tf = fwd_flops / (stage["attend_fwd"] * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": flops / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp8 scores + mxfp8 V, e4m3 P" if mxv else
                  "mxfp8 scores + bf16 P.V" if mx else w.dtype),
        "data": "synthetic (seeded normal Q/V, chunk-clustered K; no trained activations)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "C": w.C,
                   "top_k": w.top_k, "causal": w.causal, "p_max": w.p_max, "lambda": w.lam,
                   "seed": w.seed, "layout": w.description,
                   **({"outer_segments": len(w.segments) - 1, "outer_M": w.outer_M}
                      if w.segments is not None else {}),
                   **({"scores": "MXFP8 Q and K (e4m3, 32-element E8M0 blocks)"} if mx else {}),
                   **({"values": "MXFP8 V (32-key E8M0 blocks), softmax weights rounded to "
                                 "e4m3"} if mxv else {})},
        "layer_ms": ms,
        "step_ms_median": step_ms[len(step_ms) // 2],
        "step_ms_min": step_ms[0],
        "stages_ms": stage,
        "pairs": pairs,
        "pruned_fraction": 1.0 - pairs / (w.B * w.H * w.L * w.L),
        "attention_tflops": att_tf,
        "workspace_bytes": {
            "route": moc.workspace_bytes(lay, w.B, w.H, w.d, Qd.dtype, cfg, 0),
            "varlen": int(vl.ws.numel()),
            "fwd": ws_used["fwd"], "bwd": ws_used["bwd"] if with_bwd else 0,
            "attention_buffer": int(fwd_ws.numel()),
            "fwd_at_static_bound": ws_default["fwd"],
            "bwd_at_static_bound": ws_default["bwd"] if with_bwd else 0,
            "routed_rows": cap["rows"], "routed_rows_static_bound": int(vl.struct.routed_max)},
        "pool_gbs": pool_bytes / (stage["pool"] * 1e-3) / 1e9,
        "route_gbs": route_bytes / (stage["route"] * 1e-3) / 1e9,
        "gather_gbs": gather_bytes / (stage["varlen"] * 1e-3) / 1e9,
        "roofline": {
            "bound": "mfma",
            "kernel": ("attention forward with quantised scores and values (routed + anchor "
                       "kernels of moc_attend_fwd_mxv; both products on fp8)" if mxv else
                       "attention forward with quantised scores (routed + anchor kernels of "
                       "moc_attend_fwd_mx; peak weighted 2d fp8 + 2d bf16 FLOPs per pair)"
                       if mx else "attention forward (routed + anchor kernels of moc_attend_fwd)"),
            "achieved": att_tf, "peak": peak, "unit": "TFLOP/s", "frac": att_tf / peak,
            "traffic": recorded_traffic(a.workload if a.seed == 0 else ""),
            "traffic_unit": ("HBM bytes per attention-forward call: "
                             + ("" if mxv else "V transpose + ") + "routed + anchor kernels "
                             "(rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)"),
        },
        "cpu_baseline": None,
    }
    if with_bwd:
        out["backward_tflops"] = bwd_flops / (stage["attend_bwd"] * 1e-3) / 1e12
    # the same fractions against ceilings re-measured on this GPU
    mp = measured_peaks(dev)
    mpeak = (mp["mfma_fp8_tflops"] if mxv else
             4.0 / (2.0 / mp["mfma_fp8_tflops"] + 2.0 / mp["mfma_bf16_tflops"]) if mx
             else mp["mfma_bf16_tflops"])
    out["measured_peaks"] = mp
    # the probe loops are bf16 and fp8 MFMAs: an fp32 path has no measured ceiling here
    out["roofline"]["frac_of_measured_peak"] = (att_tf / mpeak if Qd.dtype != torch.float32
                                                else None)
    out["pool_hbm_frac"] = out["pool_gbs"] / PEAK_HBM_GBS
    out["route_hbm_frac"] = out["route_gbs"] / PEAK_HBM_GBS
    out["gather_hbm_frac"] = out["gather_gbs"] / PEAK_HBM_GBS
    out["pool_frac_of_measured_copy"] = out["pool_gbs"] / mp["hbm_copy_gbs"]
    out["route_frac_of_measured_copy"] = out["route_gbs"] / mp["hbm_copy_gbs"]
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, Q, K, V, a.cpu_rows)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
