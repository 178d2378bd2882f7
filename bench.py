"""Benchmark of the causal differential-attention forward path on one MI355X.

One step = one pass of the whole path on resident synthetic inputs: the causal
prefill of the Motif-2.6B-shaped layer (B=1, T=4096, H=16, d_qk=64, d_v=128,
lambda=0.8, per-head GroupNorm) followed by the split-KV decode of 64 sequences
against a 4096-long cache (H=16, 8 splits).  Both run through the C ABI on the
current torch stream; HIP events around each call time the kernels.

Prints ONE JSON line.  `value` is the prefill throughput in TFLOP/s, counting
768 FLOP per causal (query, key <= query) pair and head: two 64-wide score dot
products and two 128-wide P V products (the one-pass form has to keep P1 V and
P2 V apart).  Decode reports HBM GB/s from the bytes it must move.  The roofline
object covers the prefill kernel against the dense bf16/fp16 MFMA peak; the
cpu_baseline object times the fp64 oracle on this host's cores.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]

The default warm-up (2000 steps, about a second of GPU work) lets the GPU reach
its steady clocks before the timed region; the timed region is 200 steps.
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
ROPE_THETA = 500000.0        # Motif 2.6B's RoPE base
CSRC = os.path.join(ROOT, "differential_attention_causal_amd", "csrc")
PREFILL_PMC = os.path.join(ROOT, "profiles", "prefill_kernel_b1_t4096_h16_hbm_counters.txt")
PREFILL_SOURCES = [os.path.join(CSRC, f) for f in ("prefill.hip", "prefill_tiles.h", "kernels.h", "rope.h", "tile.h")]
DECODE_PMC = os.path.join(ROOT, "profiles", "decode_split_kernel_b64_l4096_h16_hbm_counters.txt")
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


def gpu_env(torch, clocks: bool = True) -> dict:
    """Device, software versions and current clocks (rocm-smi, when it answers;
    skipped under a profiler, which has the GPU open before the program starts,
    so that no child process is started from a process holding the GPU)."""
    import subprocess

    env = {"gpu": torch.cuda.get_device_name(0), "hip": torch.version.hip, "torch": torch.__version__}
    if not clocks:
        env["clocks"] = None
        return env
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        card = next(iter(json.loads(r.stdout).values()))
        env["clocks"] = {k: v for k, v in card.items() if "clock" in k.lower() or "sclk" in k or "mclk" in k}
    except Exception as e:  # no rocm-smi, no permission, unexpected output: report without clocks
        env["clocks"] = None
        env["clocks_error"] = type(e).__name__
    return env


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
    """Mean and minimum microseconds of fn() between events on the current stream."""
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    return float(ms.mean()) * 1e3, float(ms.min()) * 1e3


def variants(da, torch, np, to_dev, f32_dev, dev, warmup=300, iters=100):
    """The variant rows, timed after, and outside, the step's timed region:
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

    p_us, p_min = _time_calls(torch, np, prefill, warmup, iters)
    d_us, d_min = _time_calls(torch, np, decode, warmup, iters)
    r_us, r_min = _time_calls(torch, np, prefill_rope, warmup, iters)
    bw_us, bw_min = _time_calls(torch, np, backward, warmup // 3, iters)
    g_us, g_min = _time_calls(torch, np, grouped, warmup, iters)
    assert bool(torch.isfinite(gout.float()).all())
    g_flop = rw.causal_pairs * GROUPED_FLOP_PER_PAIR_HEAD  # causal_pairs already counts the 16 heads
    assert all(bool(torch.isfinite(t).all()) for t in bgr.values())
    bw_flop = rw.causal_pairs * BWD_FLOP_PER_PAIR
    assert bool(torch.isfinite(r_out.float()).all())
    r_flop = rw.causal_pairs * FLOP_PER_PAIR
    assert bool(torch.isfinite(p_out.float()).all()) and bool(torch.isfinite(d_out.float()).all())
    p_flop = pw.causal_pairs * FLOP_PER_PAIR
    d_bytes = decode_bytes(dw)
    return {
        "grouped": {"workload": "B=1 T=4096 16 heads (12 signal, 4 noise, g=3), token-wise lambda, gate",
                    "us_mean": round(g_us, 2), "us_min": round(g_min, 2),
                    "tflops": round(g_flop / g_us / 1e6, 2),
                    "frac_mfma_peak": round(g_flop / g_us / 1e6 / MFMA_PEAK_TFLOPS, 4)},
        "backward": {"workload": PREFILL_WL, "us_mean": round(bw_us, 2), "us_min": round(bw_min, 2),
                     "flop_per_pair": BWD_FLOP_PER_PAIR, "tflops": round(bw_flop / bw_us / 1e6, 2),
                     "frac_mfma_peak": round(bw_flop / bw_us / 1e6 / MFMA_PEAK_TFLOPS, 4)},
        "rope_prefill": {"workload": PREFILL_WL, "rope": "split-half", "theta": ROPE_THETA,
                         "us_mean": round(r_us, 2), "us_min": round(r_min, 2),
                         "tflops": round(r_flop / r_us / 1e6, 2),
                         "frac_mfma_peak": round(r_flop / r_us / 1e6 / MFMA_PEAK_TFLOPS, 4)},
        "prefill": {"workload": SWA_PREFILL_WL, "window": pw.window, "us_mean": round(p_us, 2),
                    "us_min": round(p_min, 2), "visible_pairs": pw.causal_pairs,
                    "tflops": round(p_flop / p_us / 1e6, 2),
                    "frac_mfma_peak": round(p_flop / p_us / 1e6 / MFMA_PEAK_TFLOPS, 4)},
        "decode": {"workload": SWA_DECODE_WL, "window": dw.window, "us_mean": round(d_us, 2),
                   "us_min": round(d_min, 2), "bytes": d_bytes, "gbs": round(d_bytes / d_us / 1e3, 1),
                   "frac_hbm_peak": round(d_bytes / d_us / 1e3 / HBM_PEAK_GBS, 4), "splits": dw.num_splits},
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the sliding-window and RoPE timings")
    ap.add_argument("--no-clocks", action="store_true", help="skip the rocm-smi clock query (for profiler runs)")
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
    torch.cuda.synchronize()

    def prefill():
        da.diffattn_fwd_prefill(P["q1"], P["q2"], P["k1"], P["k2"], P["v"], pw.lam, P["gain"], eps=pw.eps,
                                scale=pw.scale, out=p_out)

    def decode():
        da.diffattn_fwd_decode(D["q1"], D["q2"], D["k1"], D["k2"], D["v"], dw.lam, D["gain"], eps=dw.eps,
                               scale=dw.scale, num_splits=dw.num_splits, workspace=ws, out=d_out)

    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record()
        prefill()
        ev[k][1].record()
        decode()
        ev[k][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    p_ms = np.array([ev[k][0].elapsed_time(ev[k][1]) for k in range(K)])
    d_ms = np.array([ev[k][1].elapsed_time(ev[k][2]) for k in range(K)])
    step_ms = ev[0][0].elapsed_time(ev[K - 1][2]) / K
    assert bool(torch.isfinite(p_out.float()).all()) and bool(torch.isfinite(d_out.float()).all())

    var = None if args.no_variants else variants(da, torch, np, to_dev, f32_dev, dev)

    p_flop = pw.causal_pairs * FLOP_PER_PAIR
    p_s = float(p_ms.mean()) / 1e3
    tflops = p_flop / p_s / 1e12
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
                   "lambda": pw.lam, "causal": True, "step_also_runs": DECODE_WL},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": "prefill_pp_kernel", "algorithmic_flop_per_launch": p_flop},
        "prefill": {"us_mean": round(p_s * 1e6, 2), "us_min": round(float(p_ms.min()) * 1e3, 2),
                    "tflops": round(tflops, 2), "tflops_512_per_pair": round(pw.causal_pairs * 512 / p_s / 1e12, 2),
                    "frac_mfma_peak": round(tflops / MFMA_PEAK_TFLOPS, 4)},
        "decode": {"workload": DECODE_WL, "us_mean": round(d_s * 1e6, 2), "us_min": round(float(d_ms.min()) * 1e3, 2),
                   "bytes": d_bytes, "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                   "splits": dw.num_splits, "traffic": read_traffic(DECODE_PMC, DECODE_SOURCES)},
        "variants": var,
        "wall_s_timed": round(wall, 3),
        "kernel_source_sha256_16": kernel_source_digest(),
        "env": gpu_env(torch, clocks=not args.no_clocks),
    }
    if not args.no_cpu_baseline:
        # the benchmarked prefill once more (outside the timed region) with
        # fp32 and pre-norm outputs, for the parity record
        y32 = torch.empty((pw.B, pw.T, pw.H, pw.d_v), dtype=torch.float32, device=dev)
        o_pre = torch.empty_like(y32)
        da.diffattn_fwd_prefill(P["q1"], P["q2"], P["k1"], P["k2"], P["v"], pw.lam, P["gain"], eps=pw.eps,
                                scale=pw.scale, out=y32, o_pre=o_pre)
        prefill()
        torch.cuda.synchronize()
        gpu = {"y_bf16": p_out.float().cpu().numpy(), "y_f32": y32.cpu().numpy(), "o_pre": o_pre.cpu().numpy()}
        rec["cpu_baseline"] = cpu_baseline(xp, pw, gpu)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
