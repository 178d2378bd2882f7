"""rocprofv3 harness: kernel timings against the MI355X roofline, and HBM
traffic from the FETCH_SIZE / WRITE_SIZE counters, written as the text
summaries kept under profiles/.

    python3 profile_kernels.py step            # the benchmark step (prefill + decode)
    python3 profile_kernels.py variants        # one full bench run: every kernel of the step and the variants
    python3 profile_kernels.py trace NAME      # one workload (bench.py --workload NAME)
    python3 profile_kernels.py pmc NAME        # HBM counters of one workload's kernel
    python3 profile_kernels.py core NAME       # matrix-core busy, LDS and issue counters of its kernel

Every profiled program is `python3 bench.py ...`, launched directly after
rocprofv3's `--` by this process, which itself never touches the GPU.  Raw
output goes to the run-output directory OUT_REL; the summaries go to
profiles/.

Rates: prefill kernels are priced at 768 FLOP per visible (query, key) pair
and head against the dense bf16/fp16 MFMA peak (2516.6 TFLOP/s); decode and
windowed kernels by the bytes they must move against 8 TB/s (bench.py's
definitions).  Counter bytes: FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
each scaled by what the same counter reads for a plain device copy of 1 GiB
(bench.py --copy-calibration) measured in the same session.  Matrix-core
utilisation: SQ_VALU_MFMA_BUSY_CYCLES (busy cycles summed over the SIMDs)
over the dispatch's active cycles times the SIMD count, where the active
cycles are GRBM_GUI_ACTIVE, which rocprofv3 reports summed over the XCDs.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import re
import shutil
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (host-side constants and helpers only; bench imports torch lazily)

OUT_REL = os.path.join("gpurun_out", "prof")  # commands run from the repository root
OUT = os.path.join(ROOT, OUT_REL)
PROFILES = os.path.join(ROOT, "profiles")
PASS_TIMEOUT_S = 240


def _run(cmd, timeout=PASS_TIMEOUT_S):
    """Runs one command with a hard time limit; returns its stdout."""
    print("[prof] " + " ".join(cmd), flush=True)
    t0 = time.time()
    r = subprocess.run(["timeout", "-k", "10", str(timeout)] + cmd, cwd=ROOT, capture_output=True, text=True)
    print("[prof] rc=%d after %.1f s" % (r.returncode, time.time() - t0), flush=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout[-3000:] + r.stderr[-3000:])
        raise SystemExit("profiled command failed (rc=%d): %s" % (r.returncode, " ".join(cmd)))
    return r.stdout


def _rocprof(args, out_dir, program):
    if os.path.isdir(out_dir):
        shutil.rmtree(out_dir)
    rel = os.path.relpath(out_dir, ROOT)
    cmd = ["rocprofv3"] + args + ["--output-format", "csv", "-d", rel, "-o", "run", "--"] + program
    return _run(cmd), cmd


def _csv_rows(out_dir, suffix):
    paths = sorted(glob.glob(os.path.join(out_dir, "**", "*" + suffix), recursive=True))
    if not paths:
        raise SystemExit("no %s under %s" % (suffix, out_dir))
    rows = []
    for p in paths:
        with open(p, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def short_name(name: str) -> str:
    """'void diffattn::(anonymous namespace)::prefill_pp_kernel<false, false>(diffattn::PrefillArgs)'
    -> 'prefill_pp_kernel<false, false>'."""
    n = name.strip()
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):  # drop the parameter list (the last top-level parenthesis)
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not n.startswith("(anonymous", i):
            cut = i
    n = n[:cut]
    n = re.sub(r"^(?:[\w]+::|\(anonymous namespace\)::)+", "", n)
    return n


def _json_line(stdout):
    for line in reversed(stdout.splitlines()):
        line = line.strip()
        if line.startswith("{"):
            try:
                return json.loads(line)
            except ValueError:
                continue
    return {}


def _workload_rate(name):
    import synth

    wl = synth.WORKLOADS[name]
    if wl.kind == "prefill":
        flop = wl.causal_pairs * bench.FLOP_PER_PAIR
        if wl.window > 0:  # HBM-bound: bytes against 8 TB/s
            return wl, "hbm", bench.swa_prefill_bytes(wl), flop
        return wl, "mfma", flop, bench.swa_prefill_bytes(wl)
    return wl, "hbm", bench.decode_bytes(wl), wl.causal_pairs * bench.FLOP_PER_PAIR


def vtiles_bytes(wl):
    """Bytes the V^T pre-pass moves: V read (bf16), the tiles written (fp16,
    32-key tiles)."""
    return wl.B * wl.T * wl.H * wl.d_v * 2 + wl.B * wl.H * (-(-wl.T // 32)) * 32 * wl.d_v * 2


def _vtiles_roof(wl, avg):
    b = vtiles_bytes(wl)
    return "%.0f GB/s = %.4f of %.0f (HBM, %d B/launch)" % (b / avg / 1e3, b / avg / 1e3 / bench.HBM_PEAK_GBS,
                                                           bench.HBM_PEAK_GBS, b)


def _stats_table(rows):
    out = []
    for r in rows:
        out.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                    float(r["MaxNs"]) / 1e3))
    out.sort(key=lambda t: -t[1] * t[2])
    return out


def _sources_digest(kernel):
    if kernel.startswith("decode_"):
        return bench.kernel_source_digest(bench.DECODE_SOURCES), "decode.hip + kernels.h + rope.h"
    if kernel.startswith("prefill_swa"):
        files = ("window.hip", "prefill_tiles.h", "kernels.h", "rope.h", "tile.h")
        return (bench.kernel_source_digest([os.path.join(bench.CSRC, f) for f in files]), " + ".join(files))
    return bench.kernel_source_digest(), "prefill.hip + prefill_tiles.h + kernels.h + rope.h + tile.h + vtiles.hip"


def cmd_step():
    """Kernel trace of the benchmark step, next to the step's own event timings
    from an unprofiled run in the same session."""
    plain = _json_line(_run(["python3", "bench.py", "--no-cpu-baseline", "--no-variants"]))
    prog = ["python3", "bench.py", "--no-cpu-baseline", "--no-variants"]
    _, cmd = _rocprof(["--kernel-trace", "--stats"], os.path.join(OUT, "step"), prog)
    table = _stats_table(_csv_rows(os.path.join(OUT, "step"), "kernel_stats.csv"))
    pw = __import__("synth").WORKLOADS[bench.PREFILL_WL]
    dw = __import__("synth").WORKLOADS[bench.DECODE_WL]
    flop = pw.causal_pairs * bench.FLOP_PER_PAIR
    lines = ["# rocprofv3 kernel-trace summary of the benchmark step on MI355X (gfx950)",
             "# step: causal prefill %s, then decode %s (%d splits)" % (pw.name, dw.name, dw.num_splits),
             "command: " + " ".join(cmd),
             "# averages over every dispatch of the run (settle and warm-up ones included)",
             "kernel | calls | avg_us | min_us | max_us | roofline"]
    for name, calls, avg, mn, mx in table:
        roof = ""
        if name.startswith("prefill_pp_kernel"):
            roof = "%.1f TFLOP/s = %.4f of %.1f (bf16 MFMA, %d FLOP/launch)" % (
                flop / avg / 1e6, flop / avg / 1e6 / bench.MFMA_PEAK_TFLOPS, bench.MFMA_PEAK_TFLOPS, flop)
        elif name.startswith("vtiles_kernel"):
            roof = _vtiles_roof(pw, avg)
        elif name.startswith("decode_split_kernel"):
            b = bench.decode_bytes(dw)
            roof = "%.0f GB/s = %.4f of %.0f (HBM, %d B/launch, split kernel alone)" % (
                b / avg / 1e3, b / avg / 1e3 / bench.HBM_PEAK_GBS, bench.HBM_PEAK_GBS, b)
        lines.append("%s | %d | %.2f | %.2f | %.2f | %s" % (name, calls, avg, mn, mx, roof))
    lines += ["",
              "# HIP-event timings of the same command without the profiler, same session:",
              "bench_prefill_us_mean (pre-pass + kernel): %s" % plain.get("prefill", {}).get("us_mean"),
              "bench_prefill_kernel_us_mean: %s" % plain.get("prefill", {}).get("kernel_us_mean"),
              "bench_decode_us_mean (split + merge): %s" % plain.get("decode", {}).get("us_mean"),
              "bench_roofline_frac: %s" % plain.get("roofline", {}).get("frac"),
              "bench_sustained: prefill %s, decode %s" % (json.dumps(plain.get("prefill", {}).get("sustained")),
                                                        json.dumps(plain.get("decode", {}).get("sustained"))),
              "bench_sclk_mhz: %s" % json.dumps(plain.get("sclk_mhz")),
              "kernel_source_sha256_16: %s" % bench.kernel_source_digest()]
    _write("prefill_decode_step_kernel_trace.txt", lines)


def cmd_variants():
    """Kernel trace of one full bench run: the step and every variant
    (backward, RoPE, grouped prefill and decode, windowed prefill and decode,
    the larger prefills), one line per kernel."""
    prog = ["python3", "bench.py", "--no-cpu-baseline", "--steps", "20", "--warmup", "5", "--settle", "1"]
    _, cmd = _rocprof(["--kernel-trace", "--stats"], os.path.join(OUT, "variants"), prog)
    table = _stats_table(_csv_rows(os.path.join(OUT, "variants"), "kernel_stats.csv"))
    lines = ["# rocprofv3 kernel-trace summary of one full bench.py run (the step and every variant) on MI355X (gfx950)",
             "command: " + " ".join(cmd),
             "# averages over every dispatch of the run, warm-up ones included; a kernel that runs in several",
             "# variants averages over all of them (prefill_pp_kernel<false, false, true>: the step's prefill and",
             "# the B=8 and T=16384 prefills; vtiles_kernel: every workspace prefill without RoPE, prepass_kernel:",
             "# the RoPE prefill's key rotation and V^T tiles in one launch)",
             "kernel | calls | avg_us | min_us | max_us"]
    for name, calls, avg, mn, mx in table:
        lines.append("%s | %d | %.2f | %.2f | %.2f" % (name, calls, avg, mn, mx))
    lines.append("kernel_source_sha256_16: %s" % bench.kernel_source_digest())
    _write("variants_kernel_trace.txt", lines)


def cmd_trace(name):
    wl, bound, work, _ = _workload_rate(name)
    prog = ["python3", "bench.py", "--workload", name, "--steps", "50", "--warmup", "20", "--settle", "1"]
    plain = _json_line(_run(prog))
    d = os.path.join(OUT, "trace_" + name)
    _, cmd = _rocprof(["--kernel-trace", "--stats"], d, prog)
    table = _stats_table(_csv_rows(d, "kernel_stats.csv"))
    main = max((t for t in table if t[0].startswith(("prefill", "decode", "grouped", "bwd", "rope"))),
               key=lambda t: t[1] * t[2])[0]
    digest, what = _sources_digest(main)
    lines = ["# rocprofv3 kernel-trace summary of workload %s on MI355X (gfx950)" % name,
             "# B=%d T=%d H=%d window=%d" % (wl.B, wl.T, wl.H, wl.window),
             "command: " + " ".join(cmd),
             "kernel | calls | avg_us | min_us | max_us | roofline"]
    for kname, calls, avg, mn, mx in table:
        roof = ""
        if kname == main:
            if bound == "mfma":
                roof = "%.1f TFLOP/s = %.4f of %.1f (bf16 MFMA, %d FLOP/launch)" % (
                    work / avg / 1e6, work / avg / 1e6 / bench.MFMA_PEAK_TFLOPS, bench.MFMA_PEAK_TFLOPS, work)
            else:
                roof = "%.0f GB/s = %.4f of %.0f (HBM, %d B/launch)" % (
                    work / avg / 1e3, work / avg / 1e3 / bench.HBM_PEAK_GBS, bench.HBM_PEAK_GBS, work)
        elif kname.startswith("vtiles_kernel"):
            roof = _vtiles_roof(wl, avg)
        lines.append("%s | %d | %.2f | %.2f | %.2f | %s" % (kname, calls, avg, mn, mx, roof))
    lines += ["",
              "# HIP-event timing of the same command without the profiler, same session:",
              "bench_us_mean: %s" % plain.get("us_mean"),
              "bench_us_min: %s" % plain.get("us_min"),
              "# kernel sources hashed: " + what,
              "kernel_source_sha256_16: %s" % digest]
    kfile = re.sub(r"<.*", "", main)
    _write("%s_%s_kernel_trace.txt" % (kfile, name), lines)


def _counter_avgs(out_dir, counter, only_ours=True):
    """KiB per dispatch of `counter`, averaged per kernel (only this library's
    kernels unless only_ours is False)."""
    acc = {}
    for r in _csv_rows(out_dir, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        if only_ours and "diffattn" not in r["Kernel_Name"]:
            continue
        k = short_name(r["Kernel_Name"])
        v = float(r["Counter_Value"])
        key = (k, r.get("Dispatch_Id"))
        acc.setdefault(k, {}).setdefault(key, 0.0)
        acc[k][key] += v  # a counter may come split over instances; sum within a dispatch
    return {k: sum(d.values()) / len(d) for k, d in acc.items()}, {k: len(d) for k, d in acc.items()}


def cmd_pmc(name):
    wl, bound, work, _ = _workload_rate(name)
    prog = ["python3", "bench.py", "--workload", name, "--steps", "3", "--warmup", "1", "--settle", "0"]
    copy = ["python3", "bench.py", "--copy-calibration", "--steps", "3"]
    res, cmds = {}, {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        d = os.path.join(OUT, "pmc_%s_%s" % (name, counter))
        _, cmds[counter] = _rocprof(["--pmc", counter], d, prog)
        res[counter] = _counter_avgs(d, counter)
        dc = os.path.join(OUT, "copy_" + counter)
        _, cmds["copy_" + counter] = _rocprof(["--pmc", counter], dc, copy)
        res["copy_" + counter] = _counter_avgs(dc, counter, only_ours=False)
    gib_kib = float(1 << 20)  # 1 GiB in KiB

    def copy_kib(counter):
        avgs, _ = res["copy_" + counter]
        return max(avgs.values())  # the copy kernel dominates; any other dispatch is tiny

    fetch_scale = gib_kib / copy_kib("FETCH_SIZE")
    write_scale = gib_kib / copy_kib("WRITE_SIZE")
    fetch, nf = res["FETCH_SIZE"]
    write, _ = res["WRITE_SIZE"]
    main = max(fetch, key=lambda k: fetch[k] + write.get(k, 0.0))
    rd = fetch[main] * 1024 * fetch_scale
    wr = write.get(main, 0.0) * 1024 * write_scale
    alg = bench.swa_prefill_bytes(wl) if wl.kind == "prefill" else bench.decode_bytes(wl)
    digest, what = _sources_digest(main)
    lines = ["# HBM traffic of %s per dispatch, workload %s (B=%d T=%d H=%d window=%d), from two rocprofv3 --pmc "
             "passes" % (main, name, wl.B, wl.T, wl.H, wl.window),
             "command_fetch: " + " ".join(cmds["FETCH_SIZE"]),
             "command_write: " + " ".join(cmds["WRITE_SIZE"]),
             "command_copy_calibration: " + " ".join(cmds["copy_FETCH_SIZE"]).replace("FETCH_SIZE", "<counter>"),
             "dispatches_averaged: %d" % nf[main],
             "FETCH_SIZE_KiB_per_dispatch: %.1f" % fetch[main],
             "WRITE_SIZE_KiB_per_dispatch: %.1f" % write.get(main, 0.0),
             "copy_calibration: 1 GiB device copy reads FETCH_SIZE %.1f KiB and WRITE_SIZE %.1f KiB per launch" % (
                 copy_kib("FETCH_SIZE"), copy_kib("WRITE_SIZE")),
             "fetch_scale (true bytes per counted byte): %.4f" % fetch_scale,
             "write_scale: %.4f" % write_scale,
             "hbm_read_bytes_per_dispatch: %d" % rd,
             "hbm_write_bytes_per_dispatch: %d" % wr,
             "hbm_bytes_per_dispatch: %d" % (rd + wr),
             "algorithmic_bytes_per_dispatch: %d (inputs read once, bf16 output written once)" % alg,
             "traffic_over_algorithmic: %.3f" % ((rd + wr) / alg),
             "# kernel sources hashed: " + what,
             "kernel_source_sha256_16: %s" % digest]
    kfile = re.sub(r"<.*", "", main)
    _write("%s_%s_hbm_counters.txt" % (kfile, name), lines)


# Counter passes of `core` (at most 8 SQ counters and a GRBM one per pass).
CORE_PASSES = (
    ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_ANY",
     "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"),
    ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_ADDR_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS",
     "SQ_WAVES", "GRBM_GUI_ACTIVE"),
)
MI355X_XCDS = 8
MI355X_SIMDS = 4 * 256
MFMA_32X32X16_CYCLES = 32  # busy cycles per v_mfma_f32_32x32x16 (the prefill kernels' main product)


def cmd_core(name):
    wl, bound, work, _ = _workload_rate(name)
    prog = ["python3", "bench.py", "--workload", name, "--steps", "3", "--warmup", "1", "--settle", "0"]
    vals, cmds, durs = {}, [], {}
    for i, counters in enumerate(CORE_PASSES):
        d = os.path.join(OUT, "core_%s_%d" % (name, i))
        _, cmd = _rocprof(["--pmc"] + list(counters), d, prog)
        cmds.append(cmd)
        for r in _csv_rows(d, "counter_collection.csv"):
            if "diffattn" not in r["Kernel_Name"]:
                continue
            k = short_name(r["Kernel_Name"])
            key = (i, r.get("Dispatch_Id"))
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], {}).setdefault(key, 0.0)
            vals[k][r["Counter_Name"]][key] += float(r["Counter_Value"])
            durs.setdefault(k, {})[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    main = max(vals, key=lambda k: sum(durs[k].values()) / len(durs[k]))
    v = {c: sum(d.values()) / len(d) for c, d in vals[main].items()}
    dur = sum(durs[main].values()) / len(durs[main])
    active = v["GRBM_GUI_ACTIVE"] / MI355X_XCDS  # cycles per XCD
    util = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * MI355X_SIMDS)
    lds_conf = v["SQ_LDS_BANK_CONFLICT"] / max(1.0, v["SQ_LDS_IDX_ACTIVE"] - v["SQ_LDS_BANK_CONFLICT"])
    digest, what = _sources_digest(main)
    lines = ["# matrix-core, LDS and issue counters of %s per dispatch, workload %s (B=%d T=%d H=%d window=%d), "
             "from %d rocprofv3 --pmc passes" % (main, name, wl.B, wl.T, wl.H, wl.window, len(CORE_PASSES))]
    lines += ["command_%d: %s" % (i, " ".join(c)) for i, c in enumerate(cmds)]
    lines += ["%s: %.0f" % (c, v[c]) for c in sorted(v)]
    lines += ["dispatch_us_under_counters: %.2f" % (dur * 1e6),
              "active_cycles_per_xcd: %.0f (GRBM_GUI_ACTIVE / %d XCDs)" % (active, MI355X_XCDS),
              "clock_mhz_under_counters: %.0f" % (active / dur / 1e6),
              "mfma_busy_cycles_per_instruction: %.2f (SQ_VALU_MFMA_BUSY_CYCLES / SQ_INSTS_MFMA; %d for the "
              "32x32x16 product)" % (v["SQ_VALU_MFMA_BUSY_CYCLES"] / max(1.0, v["SQ_INSTS_MFMA"]),
                                     MFMA_32X32X16_CYCLES),
              "mfma_utilisation: %.4f (busy cycles / (active cycles x %d SIMDs))" % (util, MI355X_SIMDS),
              "lds_bank_conflict_cycles_per_access: %.4f" % lds_conf,
              "vector_issue_per_instruction: %.2f (SQ_ACTIVE_INST_VALU / SQ_INSTS_VALU in the counters' own units, "
              "both counting the matrix products)" % (v["SQ_ACTIVE_INST_VALU"] / max(1.0, v["SQ_INSTS_VALU"])),
              "# kernel sources hashed: " + what,
              "kernel_source_sha256_16: %s" % digest]
    kfile = re.sub(r"<.*", "", main)
    _write("%s_%s_core_counters.txt" % (kfile, name), lines)


def _write(fname, lines):
    lines = ["# made by: python3 profile_kernels.py " + " ".join(sys.argv[1:])] + lines
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, fname)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    # and a copy beside the raw output
    os.makedirs(OUT, exist_ok=True)
    shutil.copy(path, os.path.join(OUT, fname))
    print("[prof] wrote " + path, flush=True)


def main(argv):
    if len(argv) < 2 or argv[1] not in ("step", "variants", "trace", "pmc", "core"):
        print(__doc__)
        return 2
    os.makedirs(OUT, exist_ok=True)
    if argv[1] == "step":
        cmd_step()
    elif argv[1] == "variants":
        cmd_variants()
    elif argv[1] == "trace":
        for name in argv[2:]:
            cmd_trace(name)
    elif argv[1] == "pmc":
        for name in argv[2:]:
            cmd_pmc(name)
    else:
        for name in argv[2:]:
            cmd_core(name)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
