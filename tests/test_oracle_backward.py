"""Pins of the fp64 backward oracle (oracle/backward.py) against things other
than itself: the C forward oracle, finite differences, torch's own attention
and group_norm under autograd, and closed forms."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import backward as bwd
from synth.workloads import Workload


def _inputs(B=1, T=12, H=2, seed=71, d_qk=8, d_v=16, lam=0.6):
    wl = Workload("b", "prefill", B=B, T=T, H=H, seed=seed, lam=lam, d_qk=d_qk, d_v=d_v)
    x = synth.make_prefill_inputs(wl)
    x["lam"] = np.array([0.6, -0.3])[:H] if H <= 2 else np.linspace(-0.4, 0.9, H)
    x["dy"] = synth.normal_f32(seed + 1000, 9, (B, T, H, d_v)).astype(np.float64)
    return x


def _grads(x, **kw):
    a = dict(lam=x["lam"], gain=x["gain"], eps=x["eps"], scale=x["scale"], dy=x["dy"])
    a.update(kw)
    return bwd.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], a["lam"], a["gain"], a["eps"], a["scale"],
                        a["dy"])


def test_forward_matches_c_oracle():
    x = _inputs(B=2, T=20, H=2)
    g = _grads(x)
    o, y = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"], x["scale"])
    np.testing.assert_allclose(g["o"], o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(g["y"], y, rtol=0, atol=1e-11)


def test_gradients_match_central_differences():
    # Directional derivatives of the (pinned) fp64 forward along random
    # directions, against the autograd gradients.
    x = _inputs(B=1, T=9, H=2, seed=72)
    g = _grads(x)
    rng = np.random.default_rng(5)
    base = {n: bwd._f64(x[n]) for n in ("q1", "q2", "k1", "k2", "v")}
    lam = torch.tensor(x["lam"], dtype=torch.float64)
    gain = torch.tensor(np.asarray(x["gain"], np.float64))
    dy = torch.from_numpy(x["dy"])

    def f(t, lam_, gain_):
        y, _ = bwd.forward_torch(t["q1"], t["q2"], t["k1"], t["k2"], t["v"], lam_, gain_, x["eps"], x["scale"])
        return float((y * dy).sum())

    h = 1e-6
    for name in ("q1", "q2", "k1", "k2", "v"):
        d = torch.from_numpy(rng.standard_normal(base[name].shape))
        tp = dict(base, **{name: base[name] + h * d})
        tm = dict(base, **{name: base[name] - h * d})
        fd = (f(tp, lam, gain) - f(tm, lam, gain)) / (2 * h)
        an = float((torch.from_numpy(g["d" + name]) * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    d = torch.from_numpy(rng.standard_normal(2))
    fd = (f(base, lam + h * d, gain) - f(base, lam - h * d, gain)) / (2 * h)
    assert abs(fd - float((torch.from_numpy(g["dlam"]) * d).sum())) <= 1e-6 * max(1.0, abs(fd))
    d = torch.from_numpy(rng.standard_normal(gain.shape))
    fd = (f(base, lam, gain + h * d) - f(base, lam, gain - h * d)) / (2 * h)
    assert abs(fd - float((torch.from_numpy(g["dgain"]) * d).sum())) <= 1e-6 * max(1.0, abs(fd))


def test_gradient_matches_c_oracle_difference_quotient():
    # One bf16 ulp up and down of a single input element, through the C
    # oracle (which takes bf16 only): a coarse but fully independent check.
    x = _inputs(B=1, T=10, H=2, seed=73)
    g = _grads(x)
    for name, idx in (("k2", (0, 3, 1, 5)), ("q1", (0, 7, 0, 2)), ("v", (0, 4, 1, 9))):
        bits = x[name][idx]
        up, dn = x[name].copy(), x[name].copy()
        up[idx], dn[idx] = bits + 1, bits - 1  # neighbouring bf16 values (same sign, no exponent edge here)
        vals = synth.bf16_bits_to_f32(np.array([dn[idx], up[idx]], np.uint16)).astype(np.float64)

        def loss(xx):
            _, y = oracle.prefill(xx["q1"], xx["q2"], xx["k1"], xx["k2"], xx["v"], x["lam"], x["gain"], x["eps"],
                                  x["scale"])
            return float((y * x["dy"]).sum())

        fd = (loss(dict(x, **{name: up})) - loss(dict(x, **{name: dn}))) / (vals[1] - vals[0])
        an = g["d" + name][idx]
        assert abs(fd - an) <= 2e-3 * max(1.0, abs(an)), (name, fd, an)


def test_lambda0_matches_torch_sdpa_and_group_norm_autograd():
    x = _inputs(B=2, T=11, H=2, seed=74)
    g = _grads(x, lam=np.zeros(2))
    q, k, v = (bwd._f64(x[n]).permute(0, 2, 1, 3).requires_grad_(True) for n in ("q1", "k1", "v"))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=x["scale"])
    B, H, T, D = o.shape
    gain = torch.tensor(np.asarray(x["gain"], np.float64), requires_grad=True)
    y = torch.nn.functional.group_norm(o.permute(0, 2, 1, 3).reshape(B * T, H * D), H, weight=gain.reshape(-1),
                                       eps=x["eps"]).reshape(B, T, H, D)
    (y * torch.from_numpy(x["dy"])).sum().backward()
    np.testing.assert_allclose(g["dq1"], q.grad.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dk1"], k.grad.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dv"], v.grad.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dgain"], gain.grad.numpy(), rtol=0, atol=1e-11)
    assert np.all(g["dq2"] == 0) and np.all(g["dk2"] == 0)


def test_gain_gradient_closed_form():
    x = _inputs(B=2, T=13, H=2, seed=75)
    g = _grads(x)
    o, _ = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"], x["scale"])
    xhat = (o - o.mean(-1, keepdims=True)) / np.sqrt(o.var(-1, keepdims=True) + x["eps"])
    np.testing.assert_allclose(g["dgain"], (x["dy"] * xhat).sum(axis=(0, 1)), rtol=1e-10, atol=1e-12)


def test_identical_maps_cancel():
    # Along q1 = q2, k1 = k2 with lambda = 1 the output is identically 0, so
    # the gradients of the two copies cancel and V gets none.
    x = _inputs(B=1, T=10, H=2, seed=76)
    x = dict(x, q2=x["q1"], k2=x["k1"])
    g = _grads(x, lam=np.ones(2))
    np.testing.assert_allclose(g["dq1"], -g["dq2"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dk1"], -g["dk2"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dv"], 0, atol=1e-12)


# Rotary embedding and sliding window (Motif 2.6B explainer, "The block";
# picx.dev summary of the Motif 3 report, section 2.1).
VARIANTS = [dict(window=4), dict(rope=1, rope_theta=500.0, rope_pos0=3), dict(rope=2, rope_theta=50.0),
            dict(window=3, rope=1, rope_theta=1e4, rope_pos0=11)]


@pytest.mark.parametrize("var", VARIANTS)
def test_forward_variants_match_c_oracle(var):
    x = _inputs(B=2, T=14, H=2, seed=77)
    g = bwd.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"], x["scale"], x["dy"],
                     **var)
    o, y = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"], x["scale"],
                          **var)
    np.testing.assert_allclose(g["o"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["y"], y, rtol=0, atol=1e-10)


def test_rope_torch_matches_c_rotation():
    x = _inputs(B=1, T=9, H=2, seed=78)
    for mode in (1, 2):
        r = bwd.rope_torch(bwd._f64(x["q1"]), mode, 500.0, 7).numpy()
        np.testing.assert_allclose(r, oracle.rope(x["q1"], mode, 500.0, pos0=7), rtol=0, atol=1e-13)


@pytest.mark.parametrize("var", VARIANTS)
def test_variant_gradients_match_central_differences(var):
    x = _inputs(B=1, T=9, H=2, seed=79)
    g = bwd.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"], x["scale"], x["dy"],
                     **var)
    rng = np.random.default_rng(9)
    base = {n: bwd._f64(x[n]) for n in ("q1", "q2", "k1", "k2", "v")}
    lam = torch.tensor(x["lam"], dtype=torch.float64)
    gain = torch.tensor(np.asarray(x["gain"], np.float64))
    dy = torch.from_numpy(x["dy"])

    def f(t):
        y, _ = bwd.forward_torch(t["q1"], t["q2"], t["k1"], t["k2"], t["v"], lam, gain, x["eps"], x["scale"], **var)
        return float((y * dy).sum())

    h = 1e-6
    for name in ("q1", "q2", "k1", "k2", "v"):
        d = torch.from_numpy(rng.standard_normal(base[name].shape))
        fd = (f(dict(base, **{name: base[name] + h * d})) - f(dict(base, **{name: base[name] - h * d}))) / (2 * h)
        an = float((torch.from_numpy(g["d" + name]) * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


@pytest.mark.parametrize("var", [VARIANTS[0], VARIANTS[3]])
def test_variant_gradient_matches_c_oracle_difference_quotient(var):
    # As test_gradient_matches_c_oracle_difference_quotient, through the C
    # oracle's own rotation and window.
    x = _inputs(B=1, T=10, H=2, seed=80)
    g = bwd.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"], x["scale"], x["dy"],
                     **var)
    for name, idx in (("k2", (0, 3, 1, 5)), ("q1", (0, 7, 0, 2)), ("k1", (0, 6, 0, 1)), ("v", (0, 4, 1, 9))):
        bits = x[name][idx]
        up, dn = x[name].copy(), x[name].copy()
        up[idx], dn[idx] = bits + 1, bits - 1
        vals = synth.bf16_bits_to_f32(np.array([dn[idx], up[idx]], np.uint16)).astype(np.float64)

        def loss(xx):
            _, y = oracle.prefill(xx["q1"], xx["q2"], xx["k1"], xx["k2"], xx["v"], x["lam"], x["gain"], x["eps"],
                                  x["scale"], **var)
            return float((y * x["dy"]).sum())

        fd = (loss(dict(x, **{name: up})) - loss(dict(x, **{name: dn}))) / (vals[1] - vals[0])
        an = g["d" + name][idx]
        assert abs(fd - an) <= 2e-3 * max(1.0, abs(an)), (name, var, fd, an)


def test_window_covering_everything_equals_causal():
    x = _inputs(B=1, T=8, H=2, seed=81)
    a = _grads(x)
    b = bwd.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"], x["scale"], x["dy"],
                     window=8)
    for n in ("dq1", "dq2", "dk1", "dk2", "dv", "dlam", "dgain"):
        np.testing.assert_array_equal(a[n], b[n])
