"""Pins of the grouped / gated oracle (oracle.grouped; the picx.dev summary of
the Motif 3 report, section 2.2: grouped differential attention, token-wise
lambda, output gate) against things other than itself."""
from decimal import Decimal

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import Workload
from tests import bruteforce


def _heads(B, T, n_H, seed, d_qk=16, d_v=32):
    q = synth.normal_bf16(seed, 1, (B, T, n_H, d_qk))
    k = synth.normal_bf16(seed, 3, (B, T, n_H, d_qk))
    v = synth.normal_bf16(seed, 5, (B, T, n_H, d_v))
    return q, k, v


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def test_g1_shared_values_is_the_two_map_operation():
    # With g = 1 and each noise head given its signal head's values, grouped
    # attention is the Motif 2.6B operation before its GroupNorm.
    wl = Workload("g", "prefill", B=2, T=15, H=3, seed=81, lam_range=(0.2, 0.9), d_qk=16, d_v=32)
    x = synth.make_prefill_inputs(wl)
    q = np.concatenate([x["q1"], x["q2"]], axis=2)
    k = np.concatenate([x["k1"], x["k2"]], axis=2)
    v = np.concatenate([x["v"], x["v"]], axis=2)
    lam_t = np.broadcast_to(x["lam"].astype(np.float32), (2, 15, 3))
    out = oracle.grouped(q, k, v, 1, lam_t, scale=x["scale"])
    o, _ = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"].astype(np.float32), x["gain"],
                          x["eps"], x["scale"])
    np.testing.assert_allclose(out, o, rtol=0, atol=1e-13)


def test_lambda0_no_gate_is_sdpa_on_signal_heads():
    q, k, v = _heads(2, 12, 8, seed=82)  # g = 3: 6 signal heads, 2 noise heads
    out = oracle.grouped(q, k, v, 3, np.zeros((2, 12, 6), np.float32))
    qt, kt, vt = (torch.from_numpy(_f64(a)[:, :, :6]).permute(0, 2, 1, 3) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.25)
    np.testing.assert_allclose(out, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)


def test_gate():
    q, k, v = _heads(1, 10, 4, seed=83)
    lam = synth.uniform_f32(83, 7, (1, 10, 2), 0.0, 1.0)
    plain = oracle.grouped(q, k, v, 1, lam)
    half = oracle.grouped(q, k, v, 1, lam, gate=np.zeros((1, 10, 2, 32), np.float32))
    np.testing.assert_array_equal(half, 0.5 * plain)  # sigmoid(0) = 1/2 exactly
    g = synth.normal_f32(83, 8, (1, 10, 2, 32), std=3.0)
    gated = oracle.grouped(q, k, v, 1, lam, gate=g)
    np.testing.assert_allclose(gated, plain * torch.sigmoid(torch.from_numpy(g.astype(np.float64))).numpy(),
                               rtol=1e-14, atol=1e-15)


def test_repeat_g_pairs_signal_heads_with_their_noise_head():
    # g = 3, n_H = 8: signal heads 0-2 share noise head 6, 3-5 noise head 7.
    q, k, v = _heads(1, 9, 8, seed=84)
    lam = np.full((1, 9, 6), 0.7, np.float32)
    a = oracle.grouped(q, k, v, 3, lam)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 7] = synth.normal_bf16(999, 3, k2[:, :, 7].shape)
    v2[:, :, 7] = synth.normal_bf16(999, 5, v2[:, :, 7].shape)
    b = oracle.grouped(q, k2, v2, 3, lam)
    np.testing.assert_array_equal(a[:, :, :3], b[:, :, :3])
    assert np.all(np.abs(a[:, :, 3:] - b[:, :, 3:]).max(axis=(0, 1, 3)) > 1e-3)


def test_token_wise_lambda():
    q, k, v = _heads(1, 8, 4, seed=85)
    lam = np.full((1, 8, 2), 0.5, np.float32)
    a = oracle.grouped(q, k, v, 1, lam)
    lam2 = lam.copy()
    lam2[0, 5, 1] = 0.9
    b = oracle.grouped(q, k, v, 1, lam2)
    diff = np.abs(a - b).max(axis=3)
    assert diff[0, 5, 1] > 0 and np.count_nonzero(diff) == 1


@pytest.mark.parametrize("g,n_H", [(1, 2), (3, 4)])
def test_bruteforce_decimal(g, n_H):
    q, k, v = _heads(2, 7, n_H, seed=86 + g, d_qk=8, d_v=8)
    n_S = g * (n_H // (g + 1))
    lam = synth.uniform_f32(86, 7, (2, 7, n_S), 0.0, 1.0)
    gate = synth.normal_f32(86, 8, (2, 7, n_S, 8))
    out = oracle.grouped(q, k, v, g, lam, gate=gate)
    gain = np.ones((n_H, 8), np.float32)
    for b, i, s in [(0, 0, 0), (1, 6, n_S - 1), (0, 3, n_S // 2)]:
        hs, _ = bruteforce.row(q, q, k, k, v, b, i, s, 0.0, gain, 1e-5, 1 / np.sqrt(8))
        hn, _ = bruteforce.row(q, q, k, k, v, b, i, n_S + s // g, 0.0, gain, 1e-5, 1 / np.sqrt(8))
        lm = Decimal(float(lam[b, i, s]))
        for c in range(8):
            sig = 1 / (1 + (-Decimal(float(gate[b, i, s, c]))).exp())
            assert abs(out[b, i, s, c] - float((hs[c] - lm * hn[c]) * sig)) < 1e-13
