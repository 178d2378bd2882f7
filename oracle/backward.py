"""fp64 CPU oracle for the backward pass of causal differential attention.

TEST INFRASTRUCTURE ONLY: the test suite is the only caller.  Nothing here
touches the GPU, and the HIP library neither imports nor links it.

The forward it differentiates is the definition on the Motif 2.6B explainer
(section "Differential attention", figure 1 caption of "The block"), with the
same readings as the C oracle (diffattn_oracle.c): scores scaled by `scale`,
causal mask j <= i (optionally a sliding window, j > i - window), the second
map scaled by lambda (one value per head) and subtracted, times V, then a
per-head GroupNorm (biased variance, eps inside the square root, gain, no
bias); optionally the rotary embedding of Q1, Q2, K1, K2 before the scores.  It is written with plain torch fp64 ops, both
T x T maps materialised, and torch autograd supplies the gradients: the
backward pass is the calculus of that definition, nothing more.

Pins (tests/test_oracle_backward.py): the forward equals the C oracle, with
and without rope and windows; every gradient agrees with central finite
differences of the forward and with difference quotients of the C oracle's
forward (also with rope and windows);
lambda = 0 matches torch's scaled_dot_product_attention + group_norm under
autograd; the GroupNorm gain gradient has its closed form sum(dy * x_hat);
identical maps at lambda = 1 give zero attention gradients.
"""
from __future__ import annotations

import numpy as np
import torch


def _f64(bits):
    """bf16 bit patterns (np.uint16) -> fp64 tensor, exactly."""
    a = np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)
    return torch.from_numpy(a.view(np.float32).astype(np.float64))


def rope_torch(x, mode, theta, pos0=0):
    """Rotary embedding of x [B, T, H, d] (fp64 tensor, differentiable), token t
    at position pos0 + t: pair c = (i0, i1) turns by the angle
    pos * theta^(-2c/d) (Motif 2.6B explainer, section "The block": RoPE with
    base 500,000), pairing (c, c + d/2) in mode 1 and (2c, 2c + 1) in mode 2;
    mode 0 returns x."""
    if mode == 0:
        return x
    B, T, H, d = x.shape
    c = torch.arange(d // 2, dtype=torch.float64)
    pos = torch.arange(T, dtype=torch.float64) + float(pos0)
    ang = pos[:, None] * torch.pow(torch.tensor(float(theta), dtype=torch.float64), -2.0 * c / d)[None, :]
    cs, sn = torch.cos(ang)[None, :, None, :], torch.sin(ang)[None, :, None, :]
    if mode == 1:
        x0, x1 = x[..., : d // 2], x[..., d // 2:]
        return torch.cat([x0 * cs - x1 * sn, x0 * sn + x1 * cs], dim=-1)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    return torch.stack([x0 * cs - x1 * sn, x0 * sn + x1 * cs], dim=-1).reshape(B, T, H, d)


def forward_torch(q1, q2, k1, k2, v, lam, gain, eps, scale, window=0, rope=0, rope_theta=0.0, rope_pos0=0):
    """The forward in fp64 torch ops.  q*, k*: [B, T, H, d_qk]; v: [B, T, H, d_v];
    lam: [H]; gain: [H, d_v].  window > 0: query i sees keys i-window+1 .. i
    (picx.dev summary of the Motif 3 report, section 2.1), else every key
    <= i; rope: the rotary embedding of Q1, Q2, K1, K2 (rope_torch) before
    the scores.  Returns (y, o) [B, T, H, d_v]."""
    B, T, H, _ = q1.shape
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    if window > 0:
        mask &= ~torch.ones(T, T, dtype=torch.bool).tril(-window)
    q1, q2, k1, k2 = (rope_torch(t, rope, rope_theta, rope_pos0) for t in (q1, q2, k1, k2))

    def attn(q, k):
        s = torch.einsum("bihd,bjhd->bhij", q, k) * scale
        s = s.masked_fill(~mask, float("-inf"))
        return torch.softmax(s, dim=-1)

    p = attn(q1, k1) - lam.view(1, H, 1, 1) * attn(q2, k2)
    o = torch.einsum("bhij,bjhc->bihc", p, v)
    mu = o.mean(dim=-1, keepdim=True)
    var = ((o - mu) ** 2).mean(dim=-1, keepdim=True)
    y = (o - mu) / torch.sqrt(var + eps) * gain.view(1, 1, H, -1)
    return y, o


def backward(q1, q2, k1, k2, v, lam, gain, eps, scale, dy, window=0, rope=0, rope_theta=0.0, rope_pos0=0):
    """Gradients of sum(y * dy).  Inputs as the C oracle takes them (bf16 bits
    for q*, k*, v; lam scalar or [H]; gain [H, d_v] fp32 values; dy any float
    array [B, T, H, d_v]); window and rope as forward_torch takes them, the
    gradients being those of the unrotated inputs.  Returns a dict of fp64
    numpy arrays: dq1, dq2, dk1, dk2, dv, dlam ([H]), dgain ([H, d_v]), plus y
    and o."""
    H = q1.shape[2]
    lam = np.broadcast_to(np.asarray(lam, dtype=np.float64), (H,)).copy()
    t = {n: _f64(a).requires_grad_(True) for n, a in (("q1", q1), ("q2", q2), ("k1", k1), ("k2", k2), ("v", v))}
    lam_t = torch.tensor(lam, dtype=torch.float64, requires_grad=True)
    gain_t = torch.tensor(np.asarray(gain, dtype=np.float64).reshape(H, -1), requires_grad=True)
    y, o = forward_torch(t["q1"], t["q2"], t["k1"], t["k2"], t["v"], lam_t, gain_t, float(eps), float(scale),
                         window=int(window), rope=int(rope), rope_theta=float(rope_theta), rope_pos0=int(rope_pos0))
    dy_t = torch.from_numpy(np.asarray(dy, dtype=np.float64))
    (y * dy_t).sum().backward()
    out = {"d" + n: t[n].grad.numpy() for n in t}
    out["dlam"] = lam_t.grad.numpy()
    out["dgain"] = gain_t.grad.numpy()
    out["y"] = y.detach().numpy()
    out["o"] = o.detach().numpy()
    return out
