"""Benchmark of the causal differential-attention forward path on one MI355X.

One step = one pass of the whole path on resident synthetic inputs: the causal
prefill of the Motif-2.6B-shaped layer (B=1, T=4096, H=16, d_qk=64, d_v=128,
lambda=0.8, per-head GroupNorm) followed by the split-KV decode of 64 sequences
against a 4096-long cache (H=16, 8 splits).  Both run through the C ABI on the
current torch stream; HIP events around each call time the kernels.  The
prefill runs the workspace entry point (diffattn_fwd_prefill_ws): a pre-pass
converts V once into fp16 V^T tiles, and its time is inside each measured call.

Prints ONE JSON line.  `value` is the prefill throughput in TFLOP/s, counting
768 FLOP per causal (query, key <= query) pair and head: two 64-wide score dot
products and two 128-wide P V products (the one-pass form has to keep P1 V and
P2 V apart).  Decode reports HBM GB/s from the bytes it must move.  The roofline
object covers the prefill kernel against the dense bf16/fp16 MFMA peak; the
cpu_baseline object times the fp64 oracle on this host's cores.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]

Before any counted warm-up step, a time-based settle phase runs whole steps for
--settle seconds of wall clock (default 2 s, whatever --warmup says), so the GPU
reaches its steady clocks before the timed region; the shader clock is read
from sysfs right before and right after the timed region.  Then --warmup
counted steps, then --steps timed steps.
    python bench.py --copy-calibration     # plain device copy, for HBM counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = 2516.6   # MI355X dense bf16/fp16: 256 CU x 2.4 GHz x 4096 FLOP/clk/CU
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
FLOP_PER_PAIR = 768
# Backward: recomputed scores (2 x 128) + dP (256, shared by the maps since
# dO_2 = -lambda dO_1) + dV (256) + dQ (2 x 128) + dK (2 x 128) per pair.
BWD_FLOP_PER_PAIR = 1280
# Grouped attention: every head is one softmax map with its own values:
# 2 x 64 (scores) + 2 x 128 (P V) per pair and head.
GROUPED_FLOP_PER_PAIR_HEAD = 384
PREFILL_WL = "prefill_b1_t4096_h16"
DECODE_WL = "decode_b64_l4096_h16"
SWA_PREFILL_WL = "swa_b1_t16384_h16_w128"
SWA_DECODE_WL = "swa_decode_b64_l4096_h16_w128"
BATCH_WL = "batch_b8_t4096_h16"
LONGCTX_WL = "longctx_b1_t16384_h16"
ROPE_THETA = 500000.0        # Motif 2.6B's RoPE base
CSRC = os.path.join(ROOT, "differential_attention_causal_amd", "csrc")
PREFILL_PMC = os.path.join(ROOT, "profiles", "prefill_pp_kernel_prefill_b1_t4096_h16_hbm_counters.txt")
PREFILL_SOURCES = [os.path.join(CSRC, f) for f in ("prefill.hip", "prefill_tiles.h", "kernels.h", "rope.h", "tile.h",
                                                    "vtiles.hip")]
DECODE_PMC = os.path.join(ROOT, "profiles", "decode_split_kernel_decode_b64_l4096_h16_hbm_counters.txt")
DECODE_SOURCES = [os.path.join(CSRC, f) for f in ("decode.hip", "kernels.h", "rope.h")]


def kernel_source_digest(sources=PREFILL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(summary=PREFILL_PMC, sources=PREFILL_SOURCES):
    """HBM bytes per launch from a committed counter summary (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy's readings), or None when there is none
    or the kernel source changed since the counters were taken."""
    if not os.path.exists(summary):
        return None
    kv = {}
    for line in open(summary):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_digest(sources):
        return None
    try:
        return int(float(kv["hbm_bytes_per_dispatch"]))
    except (KeyError, ValueError):
        return None


def decode_bytes(wl) -> int:
    """Bytes the decode must move: the visible K1, K2, V cache positions once
    (all L, or the last `window`), both queries, the output (bf16) and the gain."""
    positions = min(wl.T, wl.window) if wl.window > 0 else wl.T
    cache = wl.B * positions * wl.H * (2 * wl.d_qk + wl.d_v) * 2
    q = 2 * wl.B * wl.H * wl.d_qk * 2
    out = wl.B * wl.H * wl.d_v * 2
    gain = wl.H * wl.d_v * 4
    return cache + q + out + gain


def grouped_decode_bytes(wl, n_signal) -> int:
    """Bytes the grouped decode must move: every head's K and V cache
    positions once, the queries, each signal head's lambda, gate (bf16) and
    output (bf16)."""
    cache = wl.B * wl.T * wl.H * (wl.d_qk + wl.d_v) * 2
    q = wl.B * wl.H * wl.d_qk * 2
    per_signal = wl.B * n_signal * (4 + 2 * wl.d_v * 2)
    return cache + q + per_signal


def swa_prefill_bytes(wl) -> int:
    """Bytes a prefill must move: Q1, Q2, K1, K2, V read once, the bf16 output
    written once, and the gain."""
    rows = wl.B * wl.T * wl.H
    return rows * (4 * wl.d_qk + wl.d_v) * 2 + rows * wl.d_v * 2 + wl.H * wl.d_v * 4


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "" where unavailable."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(x, wl, gpu=None):
    """Time the fp64 oracle on all rows of the prefill workload on this host.
    gpu: the benchmarked kernel's outputs on the same inputs (bf16 y, fp32 y,
    fp32 pre-norm o, as numpy arrays); the oracle's rows are then also the
    parity check of the measured launch configuration."""
    import numpy as np
    import oracle

    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    o_ref, y_ref = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"],
                                  x["scale"], nthreads=cores)
    dt = time.perf_counter() - t0
    flop = wl.causal_pairs * FLOP_PER_PAIR
    rec = {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "sample": "all %d rows of %s (B=1,T=4096,H=16), fp64, %.2f s wall; FLOP counted at %d per "
                     "causal pair like the GPU value" % (wl.B * wl.T * wl.H, wl.name, dt, FLOP_PER_PAIR),
           "seconds": dt, "cpu_model": cpu_model()}
    if gpu is not None:
        def ymet(y):
            d = np.abs(y.astype(np.float64) - y_ref)
            return {"y_max_abs": float(d.max()), "y_mean_abs": float(d.mean())}
        o = gpu["o_pre"].astype(np.float64)
        rec["parity"] = {"bound": {"y_max_abs": 2e-2, "y_mean_abs": 2e-3, "o_rel_f": 5e-3},
                         "bf16_out": ymet(gpu["y_bf16"]), "fp32_out": ymet(gpu["y_f32"]),
                         "o_rel_f": float(np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref))}
    return rec


def gpu_env(torch) -> dict:
    """Device and software versions (the clocks come from read_sclk_mhz)."""
    return {"gpu": torch.cuda.get_device_name(0), "hip": torch.version.hip, "torch": torch.__version__}


def read_sclk_mhz():
    """Current shader clock in MHz from sysfs (hwmon freq1_input, else the
    starred pp_dpm_sclk level), or None where neither is readable.  A file
    read: no child process, no idle gap on the GPU."""
    import glob

    for path in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/freq1_input")):
        try:
            with open(path) as f:
                return round(int(f.read().strip()) / 1e6, 1)
        except (OSError, ValueError):
            continue
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        except (OSError, ValueError, IndexError):
            continue
    return None


def settle(torch, step, seconds: float):
    """Run step() back to back until `seconds` of wall clock have passed
    (synchronising every 20 steps); returns (seconds, steps)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        n += 20
        dt = time.perf_counter() - t0
        if dt >= seconds:
            return dt, n


def copy_calibration(steps: int) -> None:
    """A plain device-to-device copy of a known size, for scaling HBM counters."""
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": steps}))


def _time_calls(torch, np, fn, warmup: int, iters: int):
    """Microseconds per call of fn() on the current stream, and the minimum of
    single calls: per call, the smaller of the back-to-back median (b2b_median,
    which the host's own time per call bounds for short kernels) and the mean
    of single calls each between its own event pair (which adds the event
    packets' dispatch latency)."""
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    b2b = b2b_median(torch, np, fn, max(20, iters // 5))
    return min(float(ms.mean()), b2b) * 1e3, float(ms.min()) * 1e3


def b2b_median(torch, np, fn, n: int, repeats: int = 5) -> float:
    """ms per call of fn: `repeats` times n back-to-back calls between two
    events on the current stream, the median of the repeats."""
    out = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / n)
    return float(np.median(out))


def variants(da, torch, np, to_dev, f32_dev, dev, warmup=300, iters=100):
    """The variant rows, timed after, and outside, the step's timed region:
    the batch (B=8, lambda per head) and long-context (T=16384) prefills,
    Motif 3's sliding-window layer type (128-token windows) as the windowed
    prefill at T=16384 and the windowed decode over the 4096-long caches, the
    T=4096 prefill with the fused RoPE prologue, the T=4096 backward, and
    the grouped form (Motif 3) on the same 16-head T=4096 shape."""
    import synth

    pw = synth.WORKLOADS[SWA_PREFILL_WL]
    dw = synth.WORKLOADS[SWA_DECODE_WL]
    xp = synth.make_prefill_inputs(pw)
    xd = synth.make_decode_inputs(dw)
    P = {n: to_dev(xp[n], dev) for n in ("q1", "q2", "k1", "k2", "v")}
    D = {n: to_dev(xd[n], dev) for n in ("q1", "q2", "k1", "k2", "v")}
    pg, dg = f32_dev(xp["gain"], dev), f32_dev(xd["gain"], dev)
    p_out = torch.empty((pw.B, pw.T, pw.H, pw.d_v), dtype=torch.bfloat16, device=dev)
    d_out = torch.empty((dw.B, dw.H, dw.d_v), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(da.diffattn_decode_workspace_bytes(dw.B, dw.H, dw.d_v, dw.num_splits), dtype=torch.uint8,
                     device=dev)

    def prefill():
        da.diffattn_fwd_prefill_ex(P["q1"], P["q2"], P["k1"], P["k2"], P["v"], pw.lam, pg, eps=pw.eps,
                                   scale=pw.scale, out=p_out, window=pw.window)

    def decode():
        da.diffattn_fwd_decode_ex(D["q1"], D["q2"], D["k1"], D["k2"], D["v"], dw.lam, dg, eps=dw.eps,
                                  scale=dw.scale, num_splits=dw.num_splits, workspace=ws, out=d_out,
                                  window=dw.window)

    # the windowed layer with RoPE in front (keys rotated once into the
    # workspace, each block's queries inside the streaming window kernel)
    pr_ws = torch.empty(da.diffattn_prefill_workspace_bytes(pw.B, pw.T, pw.H, rope=da.ROPE_HALF), dtype=torch.uint8,
                        device=dev)

    def prefill_rope_window():
        da.diffattn_fwd_prefill_ws(P["q1"], P["q2"], P["k1"], P["k2"], P["v"], pw.lam, pg, pr_ws, eps=pw.eps,
                                   scale=pw.scale, out=p_out, window=pw.window, rope=da.ROPE_HALF,
                                   rope_theta=ROPE_THETA)

    def prefill_rope():
        # the Motif 2.6B layer itself: RoPE with base 500,000 in front (keys
        # rotated once into the workspace, queries in the prefill's prologue)
        da.diffattn_fwd_prefill_ws(R["q1"], R["q2"], R["k1"], R["k2"], R["v"], rw.lam, rg, r_ws, eps=rw.eps,
                                   scale=rw.scale, out=r_out, rope=da.ROPE_HALF, rope_theta=ROPE_THETA)

    rw = synth.WORKLOADS[PREFILL_WL]
    xr = synth.make_prefill_inputs(rw)
    R = {n: to_dev(xr[n], dev) for n in ("q1", "q2", "k1", "k2", "v")}
    rg = f32_dev(xr["gain"], dev)
    r_out = torch.empty((rw.B, rw.T, rw.H, rw.d_v), dtype=torch.bfloat16, device=dev)
    r_ws = torch.empty(da.diffattn_prefill_workspace_bytes(rw.B, rw.T, rw.H, rope=da.ROPE_HALF),
                       dtype=torch.uint8, device=dev)

    # backward of the T=4096 layer: training forward once, then the timed
    # backward (dy ~ N(0,1) bf16, seeded like the inputs)
    bx = synth.make_prefill_inputs(rw)
    B_ = {n: to_dev(bx[n], dev) for n in ("q1", "q2", "k1", "k2", "v")}
    bgain = f32_dev(bx["gain"], dev)
    _, bo1, bo2, blse = da.diffattn_fwd_prefill_train(B_["q1"], B_["q2"], B_["k1"], B_["k2"], B_["v"], rw.lam, bgain,
                                                      eps=rw.eps, scale=rw.scale)
    bdy = to_dev(synth.normal_bf16(rw.seed, 9, (rw.B, rw.T, rw.H, rw.d_v)), dev)
    bws = torch.empty(da.diffattn_bwd_workspace_bytes(rw.B, rw.T, rw.H, rw.d_v), dtype=torch.uint8, device=dev)
    bgr = da.diffattn_bwd_prefill(B_["q1"], B_["q2"], B_["k1"], B_["k2"], B_["v"], rw.lam, bgain, bo1, bo2, blse, bdy,
                                  eps=rw.eps, scale=rw.scale, workspace=bws)

    def backward():
        da.diffattn_bwd_prefill(B_["q1"], B_["q2"], B_["k1"], B_["k2"], B_["v"], rw.lam, bgain, bo1, bo2, blse, bdy,
                                eps=rw.eps, scale=rw.scale, workspace=bws, grads=bgr)

    # grouped attention (Motif 3 form): 16 heads, g = 3, token-wise lambda, gate
    gq, gk = to_dev(bx["q1"], dev), to_dev(bx["k1"], dev)
    gv = B_["v"]
    glam = torch.from_numpy(synth.uniform_f32(rw.seed, 7, (rw.B, rw.T, 12), 0.0, 1.0)).to(dev)
    ggate = to_dev(synth.f32_to_bf16_bits(synth.normal_f32(rw.seed, 8, (rw.B, rw.T, 12, rw.d_v), std=2.0)), dev)
    gws = torch.empty(da.diffattn_grouped_workspace_bytes(rw.B, rw.T, rw.H, 3, rw.d_v), dtype=torch.uint8, device=dev)
    gout = torch.empty((rw.B, rw.T, 12, rw.d_v), dtype=torch.bfloat16, device=dev)

    def grouped():
        da.diffattn_fwd_grouped(gq, gk, gv, 3, glam, gate=ggate, out=gout, workspace=gws)

    # grouped decode over the decode workload's full 4096-long caches: one K and
    # one V cache per head (16 heads: 12 signal, 4 noise, g = 3)
    gdw = synth.WORKLOADS[DECODE_WL]
    gd_lam = torch.from_numpy(synth.uniform_f32(gdw.seed, 7, (gdw.B, 12), 0.0, 1.0)).to(dev)
    gd_gate = to_dev(synth.f32_to_bf16_bits(synth.normal_f32(gdw.seed, 8, (gdw.B, 12, gdw.d_v), std=2.0)), dev)
    gd_ws = torch.empty(da.diffattn_grouped_decode_workspace_bytes(gdw.B, gdw.H, gdw.d_v, 8), dtype=torch.uint8,
                        device=dev)
    gd_out = torch.empty((gdw.B, 12, gdw.d_v), dtype=torch.bfloat16, device=dev)

    def grouped_decode():
        da.diffattn_fwd_grouped_decode(D["q1"], D["k1"], D["v"], 3, gd_lam, gate=gd_gate, num_splits=8, out=gd_out,
                                       workspace=gd_ws)

    # the two other full-attention workloads: the training-shaped batch
    # (B=8, lambda per head) and the long-context layer (T=16384)
    big = {}
    for key, name in (("batch_prefill", BATCH_WL), ("longctx_prefill", LONGCTX_WL)):
        w = synth.WORKLOADS[name]
        xw = synth.make_prefill_inputs(w)
        W = {n: to_dev(xw[n], dev) for n in ("q1", "q2", "k1", "k2", "v")}
        wg = f32_dev(xw["gain"], dev)
        wl_lam = f32_dev(xw["lam"], dev) if w.lam_range is not None else w.lam
        w_out = torch.empty((w.B, w.T, w.H, w.d_v), dtype=torch.bfloat16, device=dev)
        w_ws = torch.empty(da.diffattn_prefill_workspace_bytes(w.B, w.T, w.H), dtype=torch.uint8, device=dev)

        def run(W=W, wg=wg, wl_lam=wl_lam, w_out=w_out, w=w, w_ws=w_ws):
            da.diffattn_fwd_prefill_ws(W["q1"], W["q2"], W["k1"], W["k2"], W["v"], wl_lam, wg, w_ws, eps=w.eps,
                                       scale=w.scale, out=w_out)

        us, us_min = _time_calls(torch, np, run, 60, 40)
        assert bool(torch.isfinite(w_out.float()).all())
        flop = w.causal_pairs * FLOP_PER_PAIR
        big[key] = {"workload": name, "B": w.B, "T": w.T, "H": w.H, "us_mean": round(us, 2),
                    "us_min": round(us_min, 2), "tflops": round(flop / us / 1e6, 2),
                    "frac_mfma_peak": round(flop / us / 1e6 / MFMA_PEAK_TFLOPS, 4),
                    "kernels": "vtiles_kernel + prefill_pp_kernel<false, false, true>"}
        del W, w_out, w_ws

    p_us, p_min = _time_calls(torch, np, prefill, warmup, iters)
    pr_us, pr_min = _time_calls(torch, np, prefill_rope_window, warmup, iters)
    d_us, d_min = _time_calls(torch, np, decode, warmup, iters)
    r_us, r_min = _time_calls(torch, np, prefill_rope, warmup, iters)
    bw_us, bw_min = _time_calls(torch, np, backward, warmup // 3, iters)
    g_us, g_min = _time_calls(torch, np, grouped, warmup, iters)
    gd_us, gd_min = _time_calls(torch, np, grouped_decode, warmup // 3, iters)
    assert bool(torch.isfinite(gd_out.float()).all())
    gd_bytes = grouped_decode_bytes(gdw, 12)
    assert bool(torch.isfinite(gout.float()).all())
    g_flop = rw.causal_pairs * GROUPED_FLOP_PER_PAIR_HEAD  # causal_pairs already counts the 16 heads
    assert all(bool(torch.isfinite(t).all()) for t in bgr.values())
    bw_flop = rw.causal_pairs * BWD_FLOP_PER_PAIR
    assert bool(torch.isfinite(r_out.float()).all())
    r_flop = rw.causal_pairs * FLOP_PER_PAIR
    assert bool(torch.isfinite(p_out.float()).all()) and bool(torch.isfinite(d_out.float()).all())
    p_flop = pw.causal_pairs * FLOP_PER_PAIR
    p_bytes = swa_prefill_bytes(pw)
    d_bytes = decode_bytes(dw)
    rec = dict(big)
    rec.update({
        "grouped": {"workload": "B=1 T=4096 16 heads (12 signal, 4 noise, g=3), token-wise lambda, gate",
                    "us_mean": round(g_us, 2), "us_min": round(g_min, 2),
                    "tflops": round(g_flop / g_us / 1e6, 2),
                    "frac_mfma_peak": round(g_flop / g_us / 1e6 / MFMA_PEAK_TFLOPS, 4)},
        "grouped_decode": {"workload": "B=64 L=4096 16 heads (12 signal, 4 noise, g=3), token-wise lambda, gate",
                           "bound": "hbm", "us_mean": round(gd_us, 2), "us_min": round(gd_min, 2),
                           "bytes": gd_bytes, "gbs": round(gd_bytes / gd_us / 1e3, 1),
                           "frac_hbm_peak": round(gd_bytes / gd_us / 1e3 / HBM_PEAK_GBS, 4), "splits": 8},
        "backward": {"workload": PREFILL_WL, "us_mean": round(bw_us, 2), "us_min": round(bw_min, 2),
                     "flop_per_pair": BWD_FLOP_PER_PAIR, "tflops": round(bw_flop / bw_us / 1e6, 2),
                     "frac_mfma_peak": round(bw_flop / bw_us / 1e6 / MFMA_PEAK_TFLOPS, 4)},
        "rope_prefill": {"workload": PREFILL_WL, "rope": "split-half", "theta": ROPE_THETA,
                         "kernels": "prepass_kernel + prefill_pp_kernel<false, true, true>",
                         "us_mean": round(r_us, 2), "us_min": round(r_min, 2),
                         "tflops": round(r_flop / r_us / 1e6, 2),
                         "frac_mfma_peak": round(r_flop / r_us / 1e6 / MFMA_PEAK_TFLOPS, 4)},
        # 128-key windows: 96 FLOP per algorithmic byte, below the chip's
        # ridge (about 315), so the bound is HBM
        "swa_prefill": {"workload": SWA_PREFILL_WL, "window": pw.window, "bound": "hbm",
                        "us_mean": round(p_us, 2), "us_min": round(p_min, 2), "visible_pairs": pw.causal_pairs,
                        "bytes": p_bytes, "gbs": round(p_bytes / p_us / 1e3, 1),
                        "frac_hbm_peak": round(p_bytes / p_us / 1e3 / HBM_PEAK_GBS, 4),
                        "tflops": round(p_flop / p_us / 1e6, 2)},
        # the same with RoPE: the key pre-pass (rope_keys_kernel) adds the
        # keys' fp16 copies to the bytes moved (read 2 x 64 dims, write the
        # same in fp16); priced on the algorithmic bytes of the layer itself
        "swa_rope_prefill": {"workload": SWA_PREFILL_WL, "window": pw.window, "rope": "split-half",
                             "theta": ROPE_THETA, "bound": "hbm",
                             "kernels": "rope_keys_kernel + prefill_swa_kernel<true>",
                             "us_mean": round(pr_us, 2), "us_min": round(pr_min, 2), "bytes": p_bytes,
                             "gbs": round(p_bytes / pr_us / 1e3, 1),
                             "frac_hbm_peak": round(p_bytes / pr_us / 1e3 / HBM_PEAK_GBS, 4),
                             "tflops": round(p_flop / pr_us / 1e6, 2)},
        "swa_decode": {"workload": SWA_DECODE_WL, "window": dw.window, "bound": "hbm", "us_mean": round(d_us, 2),
                       "us_min": round(d_min, 2), "bytes": d_bytes, "gbs": round(d_bytes / d_us / 1e3, 1),
                       "frac_hbm_peak": round(d_bytes / d_us / 1e3 / HBM_PEAK_GBS, 4), "splits": dw.num_splits},
    })
    return rec


def one_workload(args, da, torch, np, synth, to_dev, f32_dev) -> int:
    """Settle, warm-up and timed calls of one workload alone (a profiling
    harness target): prints {workload, kernel us_mean/us_min, rate}."""
    wl = synth.WORKLOADS[args.workload]
    dev = "cuda"
    if wl.kind == "prefill":
        x = synth.make_prefill_inputs(wl)
        t = {n: to_dev(x[n], dev) for n in ("q1", "q2", "k1", "k2", "v")}
        gain = f32_dev(x["gain"], dev)
        lam = f32_dev(x["lam"], dev) if wl.lam_range is not None else wl.lam
        out = torch.empty((wl.B, wl.T, wl.H, wl.d_v), dtype=torch.bfloat16, device=dev)
        pws = torch.empty(da.diffattn_prefill_workspace_bytes(wl.B, wl.T, wl.H), dtype=torch.uint8, device=dev)

        def call():
            # the workspace path, as the benchmark runs it (the windowed
            # streaming kernel leaves the V^T workspace unused)
            da.diffattn_fwd_prefill_ws(t["q1"], t["q2"], t["k1"], t["k2"], t["v"], lam, gain, pws, eps=wl.eps,
                                       scale=wl.scale, out=out, window=wl.window)
        work = {"flop": wl.causal_pairs * FLOP_PER_PAIR, "bytes": swa_prefill_bytes(wl)}
    else:
        x = synth.make_decode_inputs(wl)
        t = {n: to_dev(x[n], dev) for n in ("q1", "q2", "k1", "k2", "v")}
        gain = f32_dev(x["gain"], dev)
        out = torch.empty((wl.B, wl.H, wl.d_v), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(da.diffattn_decode_workspace_bytes(wl.B, wl.H, wl.d_v, wl.num_splits), dtype=torch.uint8,
                         device=dev)

        def call():
            da.diffattn_fwd_decode_ex(t["q1"], t["q2"], t["k1"], t["k2"], t["v"], wl.lam, gain, eps=wl.eps,
                                      scale=wl.scale, num_splits=wl.num_splits, workspace=ws, out=out,
                                      window=wl.window)
        work = {"flop": wl.causal_pairs * FLOP_PER_PAIR, "bytes": decode_bytes(wl)}
    settle(torch, call, args.settle)
    us, us_min = _time_calls(torch, np, call, args.warmup, args.steps)
    assert bool(torch.isfinite(out.float()).all())
    print(json.dumps({"workload": wl.name, "us_mean": round(us, 2), "us_min": round(us_min, 2),
                      "tflops": round(work["flop"] / us / 1e6, 2), "gbs": round(work["bytes"] / us / 1e3, 1),
                      "calls": args.warmup + args.steps, "settle_s": args.settle}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle", type=float, default=2.0,
                    help="seconds of back-to-back steps before the counted warm-up (clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the variant timings")
    ap.add_argument("--workload", default="",
                    help="time only this prefill or decode workload (for profiling runs); prints its own JSON line")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU only (no sharding or collectives); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration(args.steps)
        return 0

    import differential_attention_causal_amd as da
    import synth

    def to_dev(bits, device):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)

    def f32_dev(a, device):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    if args.workload:
        return one_workload(args, da, torch, np, synth, to_dev, f32_dev)

    dev = "cuda"
    pw = synth.WORKLOADS[PREFILL_WL]
    dw = synth.WORKLOADS[DECODE_WL]
    xp = synth.make_prefill_inputs(pw)
    xd = synth.make_decode_inputs(dw)
    P = {n: to_dev(xp[n], dev) for n in ("q1", "q2", "k1", "k2", "v")}
    P["gain"] = f32_dev(xp["gain"], dev)
    D = {n: to_dev(xd[n], dev) for n in ("q1", "q2", "k1", "k2", "v")}
    D["gain"] = f32_dev(xd["gain"], dev)
    p_out = torch.empty((pw.B, pw.T, pw.H, pw.d_v), dtype=torch.bfloat16, device=dev)
    d_out = torch.empty((dw.B, dw.H, dw.d_v), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(da.diffattn_decode_workspace_bytes(dw.B, dw.H, dw.d_v, dw.num_splits), dtype=torch.uint8,
                     device=dev)
    p_ws = torch.empty(da.diffattn_prefill_workspace_bytes(pw.B, pw.T, pw.H), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def prepare():
        # the workspace pre-pass: V converted once into fp16 V^T tiles (vtiles_kernel)
        da.diffattn_prefill_prepare(P["k1"], P["k2"], P["v"], p_ws)

    def prefill_kernel():
        # the ping-pong kernel alone, moving the prepared tiles by DMA
        da.diffattn_fwd_prefill_ws(P["q1"], P["q2"], P["k1"], P["k2"], P["v"], pw.lam, P["gain"], p_ws, eps=pw.eps,
                                   scale=pw.scale, out=p_out, prepared=True)

    def prefill():
        prepare()
        prefill_kernel()

    def decode():
        da.diffattn_fwd_decode(D["q1"], D["q2"], D["k1"], D["k2"], D["v"], dw.lam, D["gain"], eps=dw.eps,
                               scale=dw.scale, num_splits=dw.num_splits, workspace=ws, out=d_out)

    def step():
        prefill()
        decode()

    settle_s, settle_steps = settle(torch, step, args.settle)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    sclk_before = read_sclk_mhz()

    K = args.steps
    # events: step start | pre-pass | prefill kernel | decode (all on the current stream)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record()
        prepare()
        ev[k][1].record()
        prefill_kernel()
        ev[k][2].record()
        decode()
        ev[k][3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sclk_after = read_sclk_mhz()
    p_ms = np.array([ev[k][0].elapsed_time(ev[k][2]) for k in range(K)])  # the whole prefill call
    k1_ms = np.array([ev[k][1].elapsed_time(ev[k][2]) for k in range(K)])  # its main kernel alone
    v_ms = np.array([ev[k][0].elapsed_time(ev[k][1]) for k in range(K)])  # its V^T pre-pass
    d_ms = np.array([ev[k][2].elapsed_time(ev[k][3]) for k in range(K)])
    step_ms = ev[0][0].elapsed_time(ev[K - 1][3]) / K
    # Sustained per-call times right after the timed steps: back-to-back
    # calls of one kind between two events, median of five repeats.  They
    # leave out the dispatch latency that an event pair around a single call
    # adds (3-4 us), but a long run of the prefill alone, without the decode
    # between, may hold the shader clock lower on a power-limited part.
    n_b2b = max(20, K // 5)
    p_b2b = b2b_median(torch, np, prefill, n_b2b)  # the whole prefill call (pre-pass + kernel)
    k_b2b = b2b_median(torch, np, prefill_kernel, n_b2b)  # its main kernel alone
    d_b2b = b2b_median(torch, np, decode, n_b2b)
    assert bool(torch.isfinite(p_out.float()).all()) and bool(torch.isfinite(d_out.float()).all())

    var = None if args.no_variants else variants(da, torch, np, to_dev, f32_dev, dev)

    p_flop = pw.causal_pairs * FLOP_PER_PAIR
    p_s = float(p_ms.mean()) / 1e3
    tflops = p_flop / p_s / 1e12
    k_s = float(k1_ms.mean()) / 1e3
    k_tflops = p_flop / k_s / 1e12
    d_bytes = decode_bytes(dw)
    d_s = float(d_ms.mean()) / 1e3
    gbs = d_bytes / d_s / 1e9
    traffic = read_traffic()

    rec = {
        "metric": "diff-attn fwd TFLOP/s + % bf16 MFMA peak (T=4096,H=16); decode HBM GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PREFILL_WL, "B": pw.B, "T": pw.T, "H": pw.H, "d_qk": pw.d_qk, "d_v": pw.d_v,
                   "lambda": pw.lam, "causal": True,
                   "entry_point": "diffattn_prefill_prepare + diffattn_fwd_prefill_ws (prepared)",
                   "step_also_runs": DECODE_WL},
        # achieved: the ping-pong kernel's own launch, timed by the events
        # that bracket it inside the step (the V^T pre-pass runs just before
        # it as its own call); value: the whole prefill call, both launches;
        # traffic: the ping-pong kernel's counters
        "roofline": {"bound": "mfma", "achieved": round(k_tflops, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(k_tflops / MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": "prefill_pp_kernel<false, false, true>", "kernel_us_mean": round(k_s * 1e6, 2),
                     "timed": "prefill_pp_kernel alone (after diffattn_prefill_prepare), events in each step",
                     "algorithmic_flop_per_launch": p_flop},
        "timing": "means of one event pair per launch inside each timed step; sustained: %d back-to-back calls "
                  "of one kind between two events, median of 5 repeats, after the timed steps" % n_b2b,
        "prefill": {"us_mean": round(p_s * 1e6, 2), "us_min": round(float(p_ms.min()) * 1e3, 2),
                    "tflops": round(tflops, 2), "tflops_512_per_pair": round(pw.causal_pairs * 512 / p_s / 1e12, 2),
                    "frac_mfma_peak": round(tflops / MFMA_PEAK_TFLOPS, 4),
                    "vtiles_us_mean": round(float(v_ms.mean()) * 1e3, 2), "kernel_us_mean": round(k_s * 1e6, 2),
                    "sustained": {"us": round(p_b2b * 1e3, 2), "kernel_us": round(k_b2b * 1e3, 2)}},
        "decode": {"workload": DECODE_WL, "us_mean": round(d_s * 1e6, 2), "us_min": round(float(d_ms.min()) * 1e3, 2),
                   "bytes": d_bytes, "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                   "splits": dw.num_splits, "traffic": read_traffic(DECODE_PMC, DECODE_SOURCES),
                   "sustained": {"us": round(d_b2b * 1e3, 2)}},
        "variants": var,
        "settle_s": round(settle_s, 3),
        "settle_steps": settle_steps,
        "sclk_mhz": {"before_timed": sclk_before, "after_timed": sclk_after},
        "wall_s_timed": round(wall, 3),
        "kernel_source_sha256_16": kernel_source_digest(),
        "env": gpu_env(torch),
    }
    if not args.no_cpu_baseline:
        # the benchmarked prefill once more (outside the timed region) with
        # fp32 and pre-norm outputs, for the parity record
        y32 = torch.empty((pw.B, pw.T, pw.H, pw.d_v), dtype=torch.float32, device=dev)
        o_pre = torch.empty_like(y32)
        da.diffattn_fwd_prefill_ws(P["q1"], P["q2"], P["k1"], P["k2"], P["v"], pw.lam, P["gain"], p_ws, eps=pw.eps,
                                   scale=pw.scale, out=y32, o_pre=o_pre)
        prefill()
        torch.cuda.synchronize()
        gpu = {"y_bf16": p_out.float().cpu().numpy(), "y_f32": y32.cpu().numpy(), "o_pre": o_pre.cpu().numpy()}
        rec["cpu_baseline"] = cpu_baseline(xp, pw, gpu)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
