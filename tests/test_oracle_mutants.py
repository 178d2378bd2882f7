"""Planted mistakes: each mutant copy of the oracle's C source carries one
plausible bug, is built on the CPU, and must fail at least one of the pins
(the same checks tests/test_oracle.py applies to the real oracle).  This is
how the pins are shown to catch a dropped term, a wrong sign or index, or a
transposed operand."""
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import Workload
from tests import bruteforce

SRC = os.path.join(os.path.dirname(oracle.__file__), "diffattn_oracle.c")

MUTANTS = {
    "scale dropped": ("p1[j] = scale * a;", "p1[j] = a;"),
    "not causal": ("(int64_t)H * d_qk, (int64_t)H * d_v, i + 1 - first, d_qk, d_v,",
                   "(int64_t)H * d_qk, (int64_t)H * d_v, T - first, d_qk, d_v,"),
    "lambda sign": ("p1[j] = p1[j] - lam * p2[j];", "p1[j] = p1[j] + lam * p2[j];"),
    "second map uses K1": ("b += q2[c] * key_at(k2, j * kstride + c);",
                           "b += q2[c] * key_at(k1, j * kstride + c);"),
    "unbiased variance": ("    var /= d_v;", "    var /= (d_v - 1);"),
    "eps outside sqrt": ("double inv = 1.0 / sqrt(var + eps);", "double inv = 1.0 / (sqrt(var) + eps);"),
    "gain dropped": ("y[c] = (o[c] - mu) * inv * (double)gain[c];", "y[c] = (o[c] - mu) * inv;"),
    "lambda of head 0": ("scale, lam[h], gain + (int64_t)h * d_v, eps, p1, p2,\n                                   o_pre + r * d_v",
                         "scale, lam[0], gain + (int64_t)h * d_v, eps, p1, p2,\n                                   o_pre + r * d_v"),
    "V read with K stride": ("(int64_t)H * d_qk, (int64_t)H * d_v, i + 1 - first, d_qk, d_v,",
                             "(int64_t)H * d_qk, (int64_t)H * d_qk, i + 1 - first, d_qk, d_v,"),
    "window one key short": ("int64_t first = (window > 0 && i + 1 > window) ? i + 1 - window : 0;",
                             "int64_t first = (window > 0 && i + 1 > window) ? i + 2 - window : 0;"),
    "window ignored": ("int64_t first = (window > 0 && i + 1 > window) ? i + 1 - window : 0;",
                       "int64_t first = 0;"),
    "window keys not shifted": ("int64_t koff = ((b * T + first) * H + h) * (int64_t)d_qk;",
                                "int64_t koff = ((b * T) * H + h) * (int64_t)d_qk;"),
    "mean over wrong count": ("    mu /= d_v;", "    mu /= (d_v + 1);"),
    "second softmax short": ("    softmax_inplace(p2, n_keys);", "    softmax_inplace(p2, n_keys > 1 ? n_keys - 1 : 1);"),
    "rope not a rotation": ("x[i1] = x0 * sn + x1 * cs;", "x[i1] = -x0 * sn + x1 * cs;"),
    "rope turns backwards": ("        x[i0] = x0 * cs - x1 * sn;\n        x[i1] = x0 * sn + x1 * cs;",
                             "        x[i0] = x0 * cs + x1 * sn;\n        x[i1] = -x0 * sn + x1 * cs;"),
    "rope frequency exponent": ("pow(theta, -2.0 * c / d)", "pow(theta, -1.0 * c / d)"),
    "rope pairs adjacent in half mode": ("int i1 = mode == 1 ? c + d / 2 : 2 * c + 1;",
                                         "int i1 = mode == 1 ? 2 * c + 1 : 2 * c + 1;"),
    "rope query one position late": ("load_rotated(q1 + qoff, qa, d_qk, rope, theta, (double)(pos0 + i));",
                                     "load_rotated(q1 + qoff, qa, d_qk, rope, theta, (double)(pos0 + i + 1));"),
    "grouped repeat tiled": ("int hn_head = n_S + s / g;", "int hn_head = n_S + s % n_N;"),
    "grouped gate sign": ("d *= 1.0 / (1.0 + exp(-gv));", "d *= 1.0 / (1.0 + exp(gv));"),
    "grouped lambda of token 0": ("double l = (double)lam[(b * T + i) * n_S + s];",
                                  "double l = (double)lam[(b * T) * n_S + s];"),
    "rope decode query at n": ("load_rotated(q1 + qoff, qa, d_qk, rope, theta, (double)(pos0 + n - 1));",
                               "load_rotated(q1 + qoff, qa, d_qk, rope, theta, (double)(pos0 + n));"),
}


def _build(src_text, tmp, name):
    c = os.path.join(tmp, name + ".c")
    so = os.path.join(tmp, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-o", so, c, "-lm"])
    return oracle._bind(so)


def _inputs(B=2, T=12, H=2, seed=31, d_qk=8, d_v=16):
    wl = Workload("m", "prefill", B=B, T=T, H=H, seed=seed, lam=0.5, d_qk=d_qk, d_v=d_v)
    return synth.make_prefill_inputs(wl)


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _pins(lib):
    """Names of the pins this library fails (empty for a correct oracle)."""
    failed = []

    def run(x, lam, **kw):
        return oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], lam, x["gain"], x["eps"],
                              x["scale"], lib=lib, **kw)

    x = _inputs()
    # lambda = 0: causal SDPA + group_norm
    o, y = run(x, 0.0)
    q = torch.from_numpy(_f64(x["q1"])).permute(0, 2, 1, 3)
    k = torch.from_numpy(_f64(x["k1"])).permute(0, 2, 1, 3)
    v = torch.from_numpy(_f64(x["v"])).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=x["scale"])
    ref = ref.permute(0, 2, 1, 3).numpy()
    B, T, H, D = ref.shape
    gn = torch.nn.functional.group_norm(torch.from_numpy(ref.reshape(B * T, H * D)), H,
                                        weight=torch.from_numpy(x["gain"].astype(np.float64).reshape(-1)),
                                        eps=x["eps"]).numpy().reshape(B, T, H, D)
    if not (np.allclose(o, ref, rtol=0, atol=1e-12) and np.allclose(y, gn, rtol=0, atol=1e-10)):
        failed.append("lambda0")
    # V = ones: o = 1 - lambda_h
    lam = np.array([0.3, 0.9])
    xo = dict(x, v=np.full_like(x["v"], 0x3F80))
    o, _ = run(xo, lam)
    if not all(np.allclose(o[:, :, h], 1 - lam[h], atol=1e-12) for h in range(2)):
        failed.append("row sums")
    # brute force at T <= 16 (a few rows)
    lam = np.array([0.8, -0.4])
    o, y = run(x, lam)
    for b, i, h in [(0, 0, 0), (1, 11, 1), (0, 6, 1)]:
        ob, yb = bruteforce.row(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], b, i, h, lam[h], x["gain"],
                                x["eps"], x["scale"])
        if not (np.allclose(o[b, i, h], [float(t) for t in ob], rtol=1e-12, atol=1e-14)
                and np.allclose(y[b, i, h], [float(t) for t in yb], rtol=1e-10, atol=1e-12)):
            failed.append("brute force")
            break
    # identical maps at lambda = 1 cancel
    xi = dict(x, q2=x["q1"], k2=x["k1"])
    o, _ = run(xi, 1.0)
    if not np.all(o == 0):
        failed.append("identical maps")
    # sliding window: brute force with the window, and window 1 = (1 - lambda) v_i
    W = 4
    o, y = run(x, lam, window=W)
    for b, i, h in [(0, 2, 0), (1, 11, 1), (0, 7, 1)]:
        ob, yb = bruteforce.row(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], b, i, h, lam[h], x["gain"],
                                x["eps"], x["scale"], window=W)
        if not (np.allclose(o[b, i, h], [float(t) for t in ob], rtol=1e-12, atol=1e-14)
                and np.allclose(y[b, i, h], [float(t) for t in yb], rtol=1e-10, atol=1e-12)):
            failed.append("window brute force")
            break
    o, _ = run(x, lam, window=1)
    if not all(np.array_equal(o[:, :, h], (1.0 - lam[h]) * _f64(x["v"])[:, :, h]) for h in range(2)):
        failed.append("window 1")
    failed += _rope_pins(lib)
    failed += _grouped_pins(lib)
    return failed


def _grouped_pins(lib):
    """The grouped-attention pins of tests/test_oracle_grouped.py, compactly."""
    failed = []
    q = synth.normal_bf16(84, 1, (1, 9, 8, 8))
    k = synth.normal_bf16(84, 3, (1, 9, 8, 8))
    v = synth.normal_bf16(84, 5, (1, 9, 8, 16))
    lam = synth.uniform_f32(84, 7, (1, 9, 6), 0.0, 1.0)
    # lambda 0: SDPA on the signal heads
    out = oracle.grouped(q, k, v, 3, np.zeros_like(lam), lib=lib)
    qt, kt, vt = (torch.from_numpy(_f64(a)[:, :, :6]).permute(0, 2, 1, 3) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=8 ** -0.5)
    if not np.allclose(out, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12):
        failed.append("grouped lambda0")
    # pairing: noise head 7 feeds signal heads 3-5 only
    a = oracle.grouped(q, k, v, 3, lam, lib=lib)
    v2 = v.copy()
    v2[:, :, 7] = synth.normal_bf16(999, 5, v2[:, :, 7].shape)
    b = oracle.grouped(q, k, v2, 3, lam, lib=lib)
    if not (np.array_equal(a[:, :, :3], b[:, :, :3]) and np.all(np.abs(a[:, :, 3:] - b[:, :, 3:]).max(axis=(0, 1, 3)) > 1e-6)):
        failed.append("grouped pairing")
    # the gate against torch.sigmoid
    g = synth.normal_f32(84, 8, (1, 9, 6, 16), std=3.0)
    gated = oracle.grouped(q, k, v, 3, lam, gate=g, lib=lib)
    if not np.allclose(gated, a * torch.sigmoid(torch.from_numpy(g.astype(np.float64))).numpy(), rtol=1e-13, atol=1e-15):
        failed.append("grouped gate")
    # token-wise lambda: the difference from lambda 0 scales with each row's own lambda
    lam2 = lam.copy()
    lam2[0, 5, 1] += 0.25
    c = oracle.grouped(q, k, v, 3, lam2, lib=lib)
    d = np.abs(a - c).max(axis=3)
    if not (d[0, 5, 1] > 0 and np.count_nonzero(d) == 1):
        failed.append("grouped token lambda")
    return failed


def _rope_pins(lib):
    """The RoPE pins of tests/test_oracle.py, on 64-wide vectors."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb

    failed = []
    theta = 500000.0
    xr = synth.normal_bf16(51, 1, (1, 12, 2, 64))
    emb = LlamaRotaryEmbedding(LlamaConfig(hidden_size=128, num_attention_heads=2, head_dim=64, rope_theta=theta))
    xt = torch.from_numpy(_f64(xr)).permute(0, 2, 1, 3)
    cos, sin = emb(xt, (3 + torch.arange(12))[None])
    ref, _ = apply_rotary_pos_emb(xt, xt, cos, sin)
    got = oracle.rope(xr, 1, theta, pos0=3, lib=lib)
    if not np.allclose(got, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=2e-4):
        failed.append("rope vs transformers")
    perm = np.concatenate([np.arange(0, 64, 2), np.arange(1, 64, 2)])
    half = oracle.rope(np.ascontiguousarray(xr[..., perm]), 1, theta, pos0=3, lib=lib)
    back = np.empty_like(half)
    back[..., perm] = half
    if not np.array_equal(oracle.rope(xr, 2, theta, pos0=3, lib=lib), back):
        failed.append("rope interleaved permutation")
    # lambda = 0 prefill with RoPE is SDPA on the rotated vectors
    x = _inputs(B=1, T=10, H=2, d_qk=64, d_v=16)
    o, _ = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], 0.0, x["gain"], x["eps"], x["scale"],
                          lib=lib, rope=1, rope_theta=theta, rope_pos0=5)
    q = torch.from_numpy(oracle.rope(x["q1"], 1, theta, 5)).permute(0, 2, 1, 3)
    k = torch.from_numpy(oracle.rope(x["k1"], 1, theta, 5)).permute(0, 2, 1, 3)
    v = torch.from_numpy(_f64(x["v"])).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=x["scale"])
    if not np.allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12):
        failed.append("rope prefill sdpa")
    # decode rotates the query at position pos0 + n - 1
    n = np.array([10], np.int32)
    od, _ = oracle.decode(x["q1"][:, 9], x["q2"][:, 9], x["k1"], x["k2"], x["v"], 0.0, x["gain"], x["eps"],
                          x["scale"], seqlens=n, lib=lib, rope=1, rope_theta=theta, rope_pos0=5)
    qd = torch.from_numpy(oracle.rope(x["q1"][:, 9:10], 1, theta, 14)).permute(0, 2, 1, 3)
    kd = torch.from_numpy(_f64(x["k1"])).permute(0, 2, 1, 3)
    refd = torch.nn.functional.scaled_dot_product_attention(qd, kd, v, scale=x["scale"])
    if not np.allclose(od, refd.permute(0, 2, 1, 3).numpy()[:, 0], rtol=0, atol=1e-12):
        failed.append("rope decode position")
    return failed


def test_real_oracle_passes_all_pins():
    assert _pins(oracle._load()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation site not found: " + name
    lib = _build(src.replace(old, new), str(tmp_path), "mutant")
    assert _pins(lib), "no pin caught the planted mistake: " + name
