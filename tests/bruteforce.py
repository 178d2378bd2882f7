"""Independent scalar brute force in 40-digit decimal arithmetic (tiny T only).

Written separately from the fp64 oracle to pin it: softmax is taken as
exp(s) / sum exp(s) with no max shift, the variance as E[x^2] - E[x]^2, and
every value is a Python ``Decimal``.  The definition is the one on the Motif
2.6B explainer (section "Differential attention", figure 1 caption): two
causal softmax maps, the second scaled by lambda and subtracted, times V, then
a per-head GroupNorm with gain.
"""
from decimal import Decimal, getcontext

import numpy as np

getcontext().prec = 40


def _dec_bf16(bits):
    f = float((np.uint32(bits) << np.uint32(16)).view(np.float32))
    return Decimal(f)  # exact: every binary float is a finite decimal


def row(q1, q2, k1, k2, v, b, i, h, lam, gain, eps, scale, n_keys=None, window=0):
    """Outputs (o, y) for query row (b, i, h) as lists of Decimal.

    For decode, pass q1/q2 of shape [B, 1, H, d] and n_keys = cache length.
    window > 0 keeps only the last `window` keys of the causal range (the
    sliding-window layers in the picx.dev summary of the Motif 3 report,
    section 2.1).
    """
    n = i + 1 if n_keys is None else n_keys
    keys = range(n)[-window:] if window > 0 else range(n)
    d_qk, d_v = q1.shape[3], v.shape[3]
    sc = Decimal(float(scale))
    qi = i if n_keys is None else 0
    e1, e2 = [], []
    for j in keys:
        a = sum(_dec_bf16(q1[b, qi, h, c]) * _dec_bf16(k1[b, j, h, c]) for c in range(d_qk))
        c2 = sum(_dec_bf16(q2[b, qi, h, c]) * _dec_bf16(k2[b, j, h, c]) for c in range(d_qk))
        e1.append((sc * a).exp())
        e2.append((sc * c2).exp())
    z1, z2 = sum(e1), sum(e2)
    lm = Decimal(float(lam))
    w = [e1[t] / z1 - lm * e2[t] / z2 for t in range(len(keys))]
    o = [sum(w[t] * _dec_bf16(v[b, j, h, c]) for t, j in enumerate(keys)) for c in range(d_v)]
    mean = sum(o) / d_v
    var = sum(x * x for x in o) / d_v - mean * mean
    inv = 1 / (var + Decimal(float(eps))).sqrt()
    y = [(o[c] - mean) * inv * Decimal(float(gain[h, c])) for c in range(d_v)]
    return o, y
