"""Host-side logic of bench.py, on the CPU: the algorithmic byte and FLOP
counts it prices kernels with, the refusal of more than one GPU, and the
traffic record that turns null when the kernel sources no longer match the
counters' summary."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_bytes_of_the_decode_workload():
    # K1 + K2 + V of 64 x 4096 x 16 positions in bf16, both queries, the bf16
    # output and the fp32 gain
    wl = synth.WORKLOADS["decode_b64_l4096_h16"]
    assert bench.decode_bytes(wl) == 2147483648 + 262144 + 262144 + 8192 == 2148016128


def test_window_byte_counts():
    # a 128-token window reads only the last 128 cache positions
    dw = synth.WORKLOADS["swa_decode_b64_l4096_h16_w128"]
    assert bench.decode_bytes(dw) == 64 * 128 * 16 * (2 * 64 + 128) * 2 + 2 * 64 * 16 * 64 * 2 + 64 * 16 * 128 * 2 \
        + 16 * 128 * 4
    pw = synth.WORKLOADS["swa_b1_t16384_h16_w128"]
    rows = 16384 * 16
    assert bench.swa_prefill_bytes(pw) == rows * (4 * 64 + 128) * 2 + rows * 128 * 2 + 16 * 128 * 4 == 268443648


def test_prefill_flop_count():
    # 768 FLOP per visible (query, key) pair and head: 103.10 GFLOP at T=4096, H=16
    wl = synth.WORKLOADS["prefill_b1_t4096_h16"]
    assert wl.causal_pairs == 16 * 4096 * 4097 // 2
    assert wl.causal_pairs * bench.FLOP_PER_PAIR == 103104380928


def test_traffic_null_on_source_mismatch(tmp_path):
    summary = tmp_path / "summary.txt"
    summary.write_text("hbm_bytes_per_dispatch: 123\nkernel_source_sha256_16: 0000000000000000\n")
    assert bench.read_traffic(str(summary)) is None
    summary.write_text("hbm_bytes_per_dispatch: 123\nkernel_source_sha256_16: %s\n" % bench.kernel_source_digest())
    assert bench.read_traffic(str(summary)) == 123


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
