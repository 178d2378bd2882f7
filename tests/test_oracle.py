"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the statement it follows.  The definition comes from the Motif
2.6B explainer (section "Differential attention" and the figure 1 caption):
  o = [softmax(Q1 K1^T) - lambda softmax(Q2 K2^T)] V,  y = GroupNorm(o),
with the readings taken where the pages are silent (1/sqrt(d) scale, causal
mask, one GroupNorm group per head, biased variance, gain, no bias).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import bruteforce

WL = synth.WORKLOADS["tiny_b1_h2_t128"]


def _inputs(B=1, T=32, H=2, seed=11, d_qk=64, d_v=128):
    from synth.workloads import Workload

    wl = Workload("t", "prefill", B=B, T=T, H=H, seed=seed, lam=0.5, d_qk=d_qk, d_v=d_v)
    return synth.make_prefill_inputs(wl)


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _run(x, lam=None, **kw):
    lam = x["lam"] if lam is None else lam
    return oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], lam, x["gain"],
                          x["eps"], x["scale"], **kw)


# --- lambda = 0 is ordinary attention (explainer, "Differential attention") ---

def test_lambda0_is_causal_sdpa_plus_group_norm():
    x = _inputs(B=2, T=48, H=3)
    o, y = _run(x, lam=0.0)
    q = torch.from_numpy(_f64(x["q1"])).permute(0, 2, 1, 3)
    k = torch.from_numpy(_f64(x["k1"])).permute(0, 2, 1, 3)
    v = torch.from_numpy(_f64(x["v"])).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=x["scale"])
    ref = ref.permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    B, T, H, D = o.shape
    gn = torch.nn.functional.group_norm(torch.from_numpy(ref.reshape(B * T, H * D)), H,
                                        weight=torch.from_numpy(x["gain"].astype(np.float64).reshape(-1)),
                                        eps=x["eps"])
    np.testing.assert_allclose(y, gn.numpy().reshape(B, T, H, D), rtol=0, atol=1e-10)


def test_lambda0_ignores_second_map():
    x = _inputs(T=24)
    o, y = _run(x, lam=0.0)
    x2 = dict(x)
    x2["q2"] = synth.normal_bf16(99, 1, x["q2"].shape)
    x2["k2"] = synth.normal_bf16(99, 2, x["k2"].shape)
    o2, y2 = _run(x2, lam=0.0)
    assert np.array_equal(o, o2) and np.array_equal(y, y2)


# --- rows of the difference map sum to 1 - lambda ---

@pytest.mark.parametrize("lam", [0.0, 0.5, 0.8, 1.0, -0.3, 2.5])
def test_v_ones_gives_one_minus_lambda(lam):
    x = _inputs(T=40)
    x["v"] = np.full_like(x["v"], 0x3F80)  # bf16 1.0
    o, y = _run(x, lam=lam)
    np.testing.assert_allclose(o, 1.0 - lam, rtol=0, atol=1e-14)
    assert np.abs(y).max() < 1e-9


def test_per_head_lambda_row_sums():
    x = _inputs(T=20, H=4)
    x["v"] = np.full_like(x["v"], 0x3F80)
    lam = np.array([0.2, 0.45, 0.7, 0.9])
    o, _ = _run(x, lam=lam)
    for h in range(4):
        np.testing.assert_allclose(o[:, :, h, :], 1.0 - lam[h], rtol=0, atol=1e-14)


# --- identical maps at lambda = 1 cancel exactly ---

def test_identical_maps_lambda1_zero():
    x = _inputs(T=64)
    x["q2"], x["k2"] = x["q1"].copy(), x["k1"].copy()
    o, y = _run(x, lam=1.0)
    assert np.all(o == 0.0) and np.all(y == 0.0)


# --- independent brute force, T <= 16 ---

@pytest.mark.parametrize("T,d_qk,d_v,lam", [(16, 64, 128, 0.8), (9, 8, 16, 0.5), (5, 4, 8, -0.7)])
def test_bruteforce_decimal(T, d_qk, d_v, lam):
    x = _inputs(B=2, T=T, H=2, seed=5 + T, d_qk=d_qk, d_v=d_v)
    lam_h = np.array([lam, 0.3])
    o, y = _run(x, lam=lam_h)
    rows = [(0, 0, 0), (0, T - 1, 1), (1, T // 2, 0), (1, T - 1, 0)]
    for b, i, h in rows:
        ob, yb = bruteforce.row(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], b, i, h, lam_h[h],
                                x["gain"], x["eps"], x["scale"])
        ob = np.array([float(t) for t in ob])
        yb = np.array([float(t) for t in yb])
        np.testing.assert_allclose(o[b, i, h], ob, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(y[b, i, h], yb, rtol=1e-12, atol=1e-13)


def test_bruteforce_decimal_decode():
    from synth.workloads import Workload

    wl = Workload("d", "decode", B=2, T=7, H=2, seed=21, lam=0.8, d_qk=16, d_v=32)
    x = synth.make_decode_inputs(wl)
    seqlens = np.array([7, 4], dtype=np.int32)
    o, y = oracle.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"],
                         x["eps"], x["scale"], seqlens=seqlens)
    for b in range(2):
        for h in range(2):
            q1 = x["q1"][:, None]  # [B, 1, H, d]
            q2 = x["q2"][:, None]
            ob, yb = bruteforce.row(q1, q2, x["k1"], x["k2"], x["v"], b, 0, h, x["lam"][h],
                                    x["gain"], x["eps"], x["scale"], n_keys=int(seqlens[b]))
            np.testing.assert_allclose(o[b, h], [float(t) for t in ob], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(y[b, h], [float(t) for t in yb], rtol=1e-12, atol=1e-13)


# --- closed forms ---

def test_row0_closed_form():
    x = _inputs(B=2, T=10, H=2)
    lam = np.array([0.8, -0.25])
    o, _ = _run(x, lam=lam)
    v = _f64(x["v"])
    for h in range(2):
        np.testing.assert_allclose(o[:, 0, h], (1 - lam[h]) * v[:, 0, h], rtol=0, atol=1e-14)


def test_zero_keys_give_prefix_mean():
    x = _inputs(T=30)
    x["k1"] = np.zeros_like(x["k1"])
    x["k2"] = np.zeros_like(x["k2"])
    o, _ = _run(x, lam=0.8)
    v = _f64(x["v"])
    T = v.shape[1]
    prefix_mean = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None, None]
    np.testing.assert_allclose(o, 0.2 * prefix_mean, rtol=0, atol=1e-14)


def test_only_first_map_keys_zero():
    # K1 = 0: the first map is uniform over j <= i; the second stays a softmax.
    x = _inputs(T=12, H=1)
    x["k1"] = np.zeros_like(x["k1"])
    o, _ = _run(x, lam=0.5)
    q2, k2, v = _f64(x["q2"]), _f64(x["k2"]), _f64(x["v"])
    for i in range(12):
        s = (k2[0, : i + 1, 0] @ q2[0, i, 0]) * x["scale"]
        p = np.exp(s - s.max())
        p /= p.sum()
        ref = v[0, : i + 1, 0].mean(axis=0) - 0.5 * (p @ v[0, : i + 1, 0])
        np.testing.assert_allclose(o[0, i, 0], ref, rtol=0, atol=1e-13)


# --- invariants ---

def test_causality():
    x = _inputs(T=40)
    o, y = _run(x)
    x2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
    cut = 17
    for name in ("k1", "k2", "v", "q1", "q2"):
        x2[name][:, cut + 1:] = synth.normal_bf16(77, 3, x2[name][:, cut + 1:].shape)
    o2, y2 = _run(x2)
    assert np.array_equal(o[:, : cut + 1], o2[:, : cut + 1])
    assert np.array_equal(y[:, : cut + 1], y2[:, : cut + 1])
    assert not np.array_equal(o[:, cut + 1:], o2[:, cut + 1:])


def test_antisymmetry_lambda1():
    x = _inputs(T=25)
    o, _ = _run(x, lam=1.0)
    xs = dict(x, q1=x["q2"], k1=x["k2"], q2=x["q1"], k2=x["k1"])
    os_, _ = _run(xs, lam=1.0)
    np.testing.assert_allclose(os_, -o, rtol=0, atol=1e-15)


def test_linearity_in_v():
    x = _inputs(T=30)
    o, y = _run(x)
    x2 = dict(x, v=synth.f32_to_bf16_bits(2.0 * synth.bf16_bits_to_f32(x["v"])))
    o2, _ = _run(x2)
    assert np.array_equal(o2, 2.0 * o)  # power-of-two scaling is exact
    # GroupNorm: (2o - 2mu) / sqrt(4 var + 4 eps) == (o - mu) / sqrt(var + eps)
    _, y2 = _run(dict(x2, eps=4.0 * x["eps"]))
    np.testing.assert_allclose(y2, y, rtol=1e-13, atol=1e-13)


def test_bh_independence():
    x = _inputs(B=2, T=20, H=3)
    o, y = _run(x)
    x2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
    for name in ("q1", "q2", "k1", "k2", "v"):
        x2[name][1, :, 2] = synth.normal_bf16(55, 4, x2[name][1, :, 2].shape)
    o2, _ = _run(x2)
    mask = np.ones(o.shape[:3], bool)
    mask[1, :, 2] = False
    assert np.array_equal(o[mask], o2[mask])
    assert not np.array_equal(o[1, :, 2], o2[1, :, 2])


def test_bounds_and_norm_moments():
    x = _inputs(T=64, H=2)
    lam = 0.7
    o, _ = _run(x, lam=lam)
    v = np.abs(_f64(x["v"]))
    vmax = np.maximum.accumulate(v, axis=1)
    assert np.all(np.abs(o) <= (1 + lam) * vmax + 1e-12)
    x1 = dict(x, gain=np.ones_like(x["gain"]))
    o, y = _run(x1, lam=lam)
    mu = y.mean(axis=-1)
    var = y.var(axis=-1)
    s2 = o.var(axis=-1)
    np.testing.assert_allclose(mu, 0.0, atol=1e-12)
    np.testing.assert_allclose(var, s2 / (s2 + x["eps"]), rtol=1e-12)


def test_row_selection_matches_full():
    x = _inputs(B=2, T=33, H=2)
    o, y = _run(x)
    rows = [(1, 32, 1), (0, 0, 0), (1, 5, 0)]
    ro, ry = _run(x, rows=rows)
    for n, (b, i, h) in enumerate(rows):
        assert np.array_equal(ro[n], o[b, i, h]) and np.array_equal(ry[n], y[b, i, h])


def test_decode_equals_last_prefill_row():
    x = _inputs(B=2, T=37, H=2)
    o, y = _run(x)
    od, yd = oracle.decode(x["q1"][:, -1], x["q2"][:, -1], x["k1"], x["k2"], x["v"], x["lam"],
                           x["gain"], x["eps"], x["scale"])
    np.testing.assert_array_equal(od, o[:, -1])
    np.testing.assert_array_equal(yd, y[:, -1])
    # a shorter cached length equals the prefill row at that position
    sl = np.array([10, 37], dtype=np.int32)
    od, _ = oracle.decode(x["q1"][:, 9], x["q2"][:, 9], x["k1"], x["k2"], x["v"], x["lam"],
                          x["gain"], x["eps"], x["scale"], seqlens=sl)
    np.testing.assert_array_equal(od[0], o[0, 9])


def test_decode_empty_cache_is_zero():
    x = _inputs(B=2, T=8, H=2)
    od, yd = oracle.decode(x["q1"][:, 0], x["q2"][:, 0], x["k1"], x["k2"], x["v"], x["lam"],
                           x["gain"], x["eps"], x["scale"], seqlens=np.array([0, 3], np.int32))
    assert np.all(od[0] == 0) and np.all(yd[0] == 0) and np.any(od[1] != 0)


def test_golden_fixture():
    """Regression anchor: stored oracle values (tests/golden/make_golden.py)."""
    import json
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_rows.json")
    g = json.load(open(path))
    wl = synth.WORKLOADS[g["workload"]]
    x = synth.make_prefill_inputs(wl)
    o, y = _run(x, rows=[tuple(r) for r in g["rows"]])
    np.testing.assert_allclose(o, np.array(g["o_pre"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(y, np.array(g["y"]), rtol=0, atol=1e-13)


# --- sliding window (picx.dev summary of the Motif 3 report, section 2.1:
# sliding-window layers; query i sees the last `window` keys up to itself) ---

@pytest.mark.parametrize("window", [37, 38, 1000])
def test_window_at_least_T_is_causal(window):
    x = _inputs(B=2, T=37, H=2)
    o, y = _run(x)
    ow, yw = _run(x, window=window)
    np.testing.assert_array_equal(ow, o)
    np.testing.assert_array_equal(yw, y)


def test_window1_is_own_value():
    # one key: both softmax rows are exactly 1, so o_i = (1 - lambda_h) v_i
    x = _inputs(B=2, T=20, H=2)
    lam = np.array([0.8, -0.3])
    o, _ = _run(x, lam=lam, window=1)
    v = _f64(x["v"])
    for h in range(2):
        np.testing.assert_array_equal(o[:, :, h], (1.0 - lam[h]) * v[:, :, h])


@pytest.mark.parametrize("window", [2, 5, 11])
def test_window_bruteforce_decimal(window):
    x = _inputs(B=2, T=14, H=2, seed=41, d_qk=8, d_v=16)
    lam_h = np.array([0.7, -0.2])
    o, y = _run(x, lam=lam_h, window=window)
    for b, i, h in [(0, 0, 0), (0, window - 1, 1), (1, window, 0), (1, 13, 1), (0, 9, 0)]:
        ob, yb = bruteforce.row(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], b, i, h, lam_h[h],
                                x["gain"], x["eps"], x["scale"], window=window)
        np.testing.assert_allclose(o[b, i, h], [float(t) for t in ob], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(y[b, i, h], [float(t) for t in yb], rtol=1e-12, atol=1e-13)


def test_window_row_is_last_row_of_slice():
    # Query i under window W sees exactly what the last query of the sequence
    # slice [i-W+1, i] sees under the plain causal mask.
    x = _inputs(B=1, T=40, H=2, seed=17)
    W = 9
    o, y = _run(x, window=W)
    for i in [W - 1, W, 23, 39]:
        sl = {k: (x[k][:, i - W + 1:i + 1] if k in ("q1", "q2", "k1", "k2", "v") else x[k]) for k in x}
        os_, ys = _run(sl)
        np.testing.assert_array_equal(o[:, i], os_[:, -1])
        np.testing.assert_array_equal(y[:, i], ys[:, -1])


def test_window_decode_equals_last_prefill_row():
    x = _inputs(B=2, T=30, H=2)
    for W in [1, 7, 29, 30, 64]:
        o, y = _run(x, window=W)
        od, yd = oracle.decode(x["q1"][:, -1], x["q2"][:, -1], x["k1"], x["k2"], x["v"], x["lam"],
                               x["gain"], x["eps"], x["scale"], window=W)
        np.testing.assert_array_equal(od, o[:, -1])
        np.testing.assert_array_equal(yd, y[:, -1])
    # with a shorter cached length the window ends at that length
    o, _ = _run(x, window=5)
    od, _ = oracle.decode(x["q1"][:, 11], x["q2"][:, 11], x["k1"], x["k2"], x["v"], x["lam"],
                          x["gain"], x["eps"], x["scale"], seqlens=np.array([12, 30], np.int32), window=5)
    np.testing.assert_array_equal(od[0], o[0, 11])


def test_window_negative_rejected():
    x = _inputs(B=1, T=4, H=2)
    with pytest.raises(RuntimeError):
        _run(x, window=-1)


# --- ring-buffer cache for sliding-window decode: a cache of L slots keeps
# the last L positions, position p in slot p % L ---

def _ring_from_linear(t, n, L):
    """Ring image of a linear [B, N, H, D] cache after n[b] positions."""
    B = t.shape[0]
    r = np.zeros((B, L) + t.shape[2:], t.dtype)
    for b in range(B):
        for p in range(int(n[b])):
            r[b, p % L] = t[b, p]
    return r


def test_ring_matches_linear_cache():
    from synth.workloads import Workload

    L, N = 8, 40
    wl = Workload("r", "decode", B=5, T=N, H=2, seed=33, lam=0.6, d_qk=16, d_v=32)
    x = synth.make_decode_inputs(wl)
    n = np.array([3, 8, 9, 21, 40], np.int32)
    ring = {k: _ring_from_linear(x[k], n, L) for k in ("k1", "k2", "v")}
    for W in [0, 1, 3, 7, 8]:
        o_r, y_r = oracle.decode(x["q1"], x["q2"], ring["k1"], ring["k2"], ring["v"], x["lam"], x["gain"],
                                 x["eps"], x["scale"], seqlens=n, window=W, ring=True)
        o_l, y_l = oracle.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"],
                                 x["eps"], x["scale"], seqlens=n, window=W if W else L)
        np.testing.assert_array_equal(o_r, o_l)
        np.testing.assert_array_equal(y_r, y_l)


def test_ring_without_wrap_is_linear():
    from synth.workloads import Workload

    wl = Workload("r", "decode", B=3, T=12, H=2, seed=34, lam=0.6, d_qk=16, d_v=32)
    x = synth.make_decode_inputs(wl)
    n = np.array([0, 5, 12], np.int32)
    for W in [0, 4]:
        a = oracle.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"],
                          x["scale"], seqlens=n, window=W, ring=True)
        b = oracle.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"],
                          x["scale"], seqlens=n, window=W)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])
    with pytest.raises(RuntimeError):
        oracle.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"],
                      x["scale"], seqlens=n, window=13, ring=True)


# --- rotary position embedding (Motif 2.6B explainer, section "The block":
# RoPE with base 500,000).  The pairing is a reading: split-half pairs
# (c, c + 32) as in the Hugging Face Llama code, or interleaved pairs
# (2c, 2c + 1); each 64-wide Q1, Q2, K1, K2 vector is rotated on its own. ---

THETA = 500000.0


def _rope_x(B=2, T=40, H=2, d=64, seed=51):
    return synth.normal_bf16(seed, 1, (B, T, H, d))


def test_rope_half_matches_transformers_llama():
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb

    x = _rope_x()
    B, T, H, d = x.shape
    cfg = LlamaConfig(hidden_size=H * d, num_attention_heads=H, head_dim=d, rope_theta=THETA)
    emb = LlamaRotaryEmbedding(cfg)
    pos0 = 7
    xt = torch.from_numpy(_f64(x)).permute(0, 2, 1, 3)  # [B, H, T, d]
    cos, sin = emb(xt, (pos0 + torch.arange(T))[None].expand(B, T))
    ref, _ = apply_rotary_pos_emb(xt, xt, cos, sin)
    got = oracle.rope(x, oracle.ROPE_HALF, THETA, pos0=pos0)
    # the library forms its angles in fp32: about 1e-5 at these positions
    np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=2e-4)


def test_rope_interleaved_is_half_on_permuted_dims():
    # Interleaved pair (2c, 2c+1) is split-half pair (c, c+32) after moving
    # dim 2c to c and dim 2c+1 to c+32.
    x = _rope_x()
    perm = np.concatenate([np.arange(0, 64, 2), np.arange(1, 64, 2)])
    half = oracle.rope(np.ascontiguousarray(x[..., perm]), oracle.ROPE_HALF, THETA, pos0=3)
    inter = oracle.rope(x, oracle.ROPE_INTERLEAVED, THETA, pos0=3)
    back = np.empty_like(half)
    back[..., perm] = half
    np.testing.assert_array_equal(inter, back)


@pytest.mark.parametrize("mode", [1, 2])
def test_rope_closed_forms(mode):
    x = _rope_x(B=1, T=1, H=1)
    xf = _f64(x)[0, 0, 0]
    # position 0 is the identity
    np.testing.assert_array_equal(oracle.rope(x, mode, THETA, pos0=0)[0, 0, 0], xf)
    # pair 0 turns by exactly `pos` radians (frequency theta^0 = 1)
    i0, i1 = (0, 32) if mode == 1 else (0, 1)
    for pos in (1, 2, 100, 12345, 1 << 20):
        r = oracle.rope(x, mode, THETA, pos0=pos)[0, 0, 0]
        c, s = math.cos(pos), math.sin(pos)
        assert abs(r[i0] - (xf[i0] * c - xf[i1] * s)) < 1e-12
        assert abs(r[i1] - (xf[i0] * s + xf[i1] * c)) < 1e-12
    # the last pair turns by pos * theta^(-62/64)
    j0, j1 = (31, 63) if mode == 1 else (62, 63)
    pos = 5000
    a = pos * THETA ** (-62 / 64)
    r = oracle.rope(x, mode, THETA, pos0=pos)[0, 0, 0]
    assert abs(r[j0] - (xf[j0] * math.cos(a) - xf[j1] * math.sin(a))) < 1e-12


@pytest.mark.parametrize("mode", [1, 2])
def test_rope_is_a_rotation_by_relative_position(mode):
    q = _rope_x(B=1, T=1, H=3, seed=52)
    k = _rope_x(B=1, T=1, H=3, seed=53)
    qf, kf = _f64(q), _f64(k)
    # each pair keeps its length
    rq = oracle.rope(q, mode, THETA, pos0=777)
    pairs = (lambda a: (a[..., :32], a[..., 32:])) if mode == 1 else (lambda a: (a[..., 0::2], a[..., 1::2]))
    a0, a1 = pairs(rq)
    b0, b1 = pairs(qf)
    np.testing.assert_allclose(a0 ** 2 + a1 ** 2, b0 ** 2 + b1 ** 2, rtol=1e-12)
    # scores depend only on the distance between the two positions
    def score(pq, pk):
        return np.sum(oracle.rope(q, mode, THETA, pos0=pq) * oracle.rope(k, mode, THETA, pos0=pk), axis=-1)
    ref = score(40, 13)
    for shift in (1, 1000, 300000):
        np.testing.assert_allclose(score(40 + shift, 13 + shift), ref, rtol=0, atol=1e-10)
    assert np.abs(score(41, 13) - ref).max() > 1e-3


def test_rope_pos_start_per_batch_row():
    x = _rope_x(B=3, T=5, H=2)
    got = oracle.rope(x, 1, THETA, pos0=10, pos_start=np.array([0, 4, 100]))
    for b, st in enumerate((0, 4, 100)):
        np.testing.assert_array_equal(got[b], oracle.rope(x[b:b + 1], 1, THETA, pos0=10 + st)[0])


@pytest.mark.parametrize("mode", [1, 2])
def test_rope_prefill_lambda0_is_sdpa_on_rotated(mode):
    x = _inputs(B=2, T=33, H=2)
    pos0 = 11
    o, y = _run(x, lam=0.0, rope=mode, rope_theta=THETA, rope_pos0=pos0)
    q = torch.from_numpy(oracle.rope(x["q1"], mode, THETA, pos0)).permute(0, 2, 1, 3)
    k = torch.from_numpy(oracle.rope(x["k1"], mode, THETA, pos0)).permute(0, 2, 1, 3)
    v = torch.from_numpy(_f64(x["v"])).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=x["scale"])
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", [1, 2])
def test_rope_prefill_shift_invariant(mode):
    # every score depends on i - j only, so moving all tokens changes nothing
    x = _inputs(B=1, T=30, H=2)
    a = _run(x, rope=mode, rope_theta=THETA, rope_pos0=0)
    b = _run(x, rope=mode, rope_theta=THETA, rope_pos0=4321)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-10)
    c = _run(x)
    assert np.abs(a[0] - c[0]).max() > 1e-3  # and it is not the plain result


@pytest.mark.parametrize("mode", [1, 2])
def test_rope_decode_rotates_query_at_last_position(mode):
    from synth.workloads import Workload

    wl = Workload("d", "decode", B=3, T=20, H=2, seed=61, lam=0.0)
    x = synth.make_decode_inputs(wl)
    n = np.array([20, 7, 1], np.int32)
    pos0 = 5
    o, _ = oracle.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], 0.0, x["gain"], x["eps"], x["scale"],
                         seqlens=n, rope=mode, rope_theta=THETA, rope_pos0=pos0)
    for b in range(3):
        q = oracle.rope(x["q1"][b:b + 1, None], mode, THETA, pos0 + int(n[b]) - 1)[0, 0]  # [H, d]
        k = _f64(x["k1"][b, : n[b]])  # cache used as given
        v = _f64(x["v"][b, : n[b]])
        for h in range(2):
            s = k[:, h] @ q[h] * x["scale"]
            p = np.exp(s - s.max())
            p /= p.sum()
            np.testing.assert_allclose(o[b, h], p @ v[:, h], rtol=0, atol=1e-12)


def test_rope_rejects_bad_arguments():
    x = _inputs(B=1, T=4, H=2)
    with pytest.raises(ValueError):
        _run(x, rope=3, rope_theta=THETA)
    with pytest.raises(ValueError):
        _run(x, rope=1, rope_theta=0.0)
