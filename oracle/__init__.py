"""fp64 CPU oracle for causal differential attention (forward).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The HIP library neither
imports nor links anything here, and nothing here touches the GPU.

The arithmetic lives in ``diffattn_oracle.c`` (plain C, fp64, OpenMP over
rows); this module only builds it, marshals numpy arrays and returns fp64
results.  See that file's header for the definition it follows and the
readings taken where the pages are silent.

Pins (tests/test_oracle.py): lambda = 0 against torch's causal scaled dot
product attention and group_norm in fp64; rows of the difference map summing
to 1 - lambda (V = ones); the all-zero output of identical maps at lambda = 1;
an independent 40-digit ``decimal`` brute force for T <= 16; closed forms for
row 0 and for zero keys; causality, antisymmetry, linearity and (b, h)
independence; decode equal to the last prefill row.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", _LIB_PATH,
           os.path.join(_HERE, "diffattn_oracle.c"), "-lm"]
    subprocess.check_call(cmd)
    return _LIB_PATH


def _bind(path):
    """ctypes handle of an oracle library at `path` (the tests also bind
    deliberately broken copies, to check that the pins catch them)."""
    lib = ctypes.CDLL(path)
    P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    lib.oracle_prefill.restype = I
    I64 = ctypes.c_int64
    lib.oracle_prefill.argtypes = [P, P, P, P, P, I, I, I, I, I, P, P, D, D, I, I, D, I64, P,
                                   I64, P, P, I]
    lib.oracle_decode.restype = I
    lib.oracle_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P, D, D, I, I, I, D, I64, P, P, I]
    lib.oracle_grouped.restype = I
    lib.oracle_grouped.argtypes = [P, P, P, I, I, I, I, I, I, P, P, D, P, I64, P, I]
    lib.oracle_rope.restype = I
    lib.oracle_rope.argtypes = [P, P, I, I, I, I, I, D, I64, P]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(_LIB_PATH)
    return _lib


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (np.uint16)")
    return a


def _lam(lam, H):
    lam = np.asarray(lam, dtype=np.float64)
    if lam.ndim == 0:
        lam = np.full((H,), float(lam))
    if lam.shape != (H,):
        raise ValueError("lambda must be a scalar or have shape [H]")
    return np.ascontiguousarray(lam)


ROPE_NONE, ROPE_HALF, ROPE_INTERLEAVED = 0, 1, 2


def _rope_args(rope, theta):
    rope = int(rope)
    if rope not in (ROPE_NONE, ROPE_HALF, ROPE_INTERLEAVED):
        raise ValueError("rope must be 0 (none), 1 (split-half) or 2 (interleaved)")
    if rope and not float(theta) > 0:
        raise ValueError("rope_theta must be > 0")
    return rope, float(theta)


def rope(x, mode, theta, pos0=0, pos_start=None, lib=None):
    """Rotary embedding of bf16 bits x [B, T, H, d] in fp64: token t of batch
    row b at position pos0 + pos_start[b] + t (pos_start optional).  Returns
    the rotated fp64 array."""
    x = _u16(x)
    B, T, H, d = x.shape
    mode, theta = _rope_args(mode, theta)
    ps = None if pos_start is None else np.ascontiguousarray(pos_start, dtype=np.int32).reshape(B)
    out = np.empty(x.shape, dtype=np.float64)
    rc = (lib or _load()).oracle_rope(x.ctypes.data, out.ctypes.data, B, T, H, d, mode, theta, int(pos0),
                                      None if ps is None else ps.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_rope failed")
    return out


def prefill(q1, q2, k1, k2, v, lam, gain, eps, scale, rows=None, nthreads=0, lib=None, window=0,
            rope=ROPE_NONE, rope_theta=0.0, rope_pos0=0):
    """Causal prefill in fp64.

    q1, q2, k1, k2: bf16 bits [B, T, H, d_qk]; v: bf16 bits [B, T, H, d_v].
    lam: scalar or [H]; gain: [H, d_v] (fp32 values); eps, scale: floats.
    rows: optional sequence of (b, i, h) triples; default all rows.
    window: > 0 for a sliding window of that many keys (query i sees
    i-window+1 .. i), 0 for every key <= i.
    rope: ROPE_HALF or ROPE_INTERLEAVED rotates Q1, Q2, K1, K2 (base
    rope_theta), token t at position rope_pos0 + t.
    Returns (o_pre, y) as fp64 arrays of shape [B, T, H, d_v], or [n_rows, d_v]
    when rows are given.
    """
    q1, q2, k1, k2, v = (_u16(a) for a in (q1, q2, k1, k2, v))
    B, T, H, d_qk = q1.shape
    d_v = v.shape[3]
    for a in (q2, k1, k2):
        if a.shape != q1.shape:
            raise ValueError("q1, q2, k1, k2 must share one shape")
    if v.shape[:3] != (B, T, H):
        raise ValueError("v must be [B, T, H, d_v]")
    gain = np.ascontiguousarray(gain, dtype=np.float32).reshape(H, d_v)
    lam = _lam(lam, H)
    rope, rope_theta = _rope_args(rope, rope_theta)
    if rows is None:
        flat = None
        n = B * T * H
    else:
        r = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
        if ((r[:, 0] < 0) | (r[:, 0] >= B) | (r[:, 1] < 0) | (r[:, 1] >= T) |
                (r[:, 2] < 0) | (r[:, 2] >= H)).any():
            raise ValueError("row index out of range")
        flat = np.ascontiguousarray((r[:, 0] * T + r[:, 1]) * H + r[:, 2])
        n = flat.shape[0]
    o = np.empty((n, d_v), dtype=np.float64)
    y = np.empty((n, d_v), dtype=np.float64)
    rc = (lib or _load()).oracle_prefill(q1.ctypes.data, q2.ctypes.data, k1.ctypes.data, k2.ctypes.data,
                                v.ctypes.data, B, T, H, d_qk, d_v, lam.ctypes.data,
                                gain.ctypes.data, float(eps), float(scale), int(window),
                                rope, rope_theta, int(rope_pos0),
                                None if flat is None else flat.ctypes.data, n,
                                o.ctypes.data, y.ctypes.data, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_prefill failed")
    if rows is None:
        return o.reshape(B, T, H, d_v), y.reshape(B, T, H, d_v)
    return o, y


def decode(q1, q2, k1, k2, v, lam, gain, eps, scale, seqlens=None, nthreads=0, lib=None, window=0, ring=False,
           rope=ROPE_NONE, rope_theta=0.0, rope_pos0=0):
    """Single-query decode in fp64: q [B, H, d_qk] against caches [B, L, H, d].

    seqlens: optional [B] cached lengths (above L counts as L; <= 0 gives zeros).
    window: > 0 attends only the last `window` positions.
    ring: the L cache slots are a ring buffer (position p in slot p % L;
    seqlens may exceed L; window 0 means L; window > L is an error).
    rope: rotates q1, q2 at position rope_pos0 + n - 1 (n = the sequence's
    length); the cache is taken as already rotated.
    Returns (o_pre, y), fp64 [B, H, d_v].
    """
    q1, q2, k1, k2, v = (_u16(a) for a in (q1, q2, k1, k2, v))
    B, H, d_qk = q1.shape
    L = k1.shape[1]
    d_v = v.shape[3]
    if q2.shape != q1.shape or k1.shape != (B, L, H, d_qk) or k2.shape != k1.shape \
            or v.shape[:3] != (B, L, H):
        raise ValueError("decode shapes disagree")
    gain = np.ascontiguousarray(gain, dtype=np.float32).reshape(H, d_v)
    lam = _lam(lam, H)
    rope, rope_theta = _rope_args(rope, rope_theta)
    sl = None
    if seqlens is not None:
        sl = np.ascontiguousarray(seqlens, dtype=np.int32)
        if sl.shape != (B,):
            raise ValueError("seqlens must be [B]")
    o = np.empty((B, H, d_v), dtype=np.float64)
    y = np.empty((B, H, d_v), dtype=np.float64)
    rc = (lib or _load()).oracle_decode(q1.ctypes.data, q2.ctypes.data, k1.ctypes.data, k2.ctypes.data,
                               v.ctypes.data, None if sl is None else sl.ctypes.data,
                               B, L, H, d_qk, d_v, lam.ctypes.data, gain.ctypes.data,
                               float(eps), float(scale), int(window), int(bool(ring)), rope, rope_theta,
                               int(rope_pos0), o.ctypes.data,
                               y.ctypes.data,
                               int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_decode failed")
    return o, y


def grouped(q, k, v, group, lam, gate=None, scale=None, rows=None, nthreads=0, lib=None):
    """Grouped differential attention with token-wise lambda and output gate,
    in fp64 (see oracle_grouped in diffattn_oracle.c for the definition and
    the readings).  q, k: bf16 bits [B, T, n_H, d_qk]; v: [B, T, n_H, d_v];
    group: g (n_N = n_H / (g + 1) noise heads, n_S = g n_N signal heads);
    lam: [B, T, n_S]; gate: optional [B, T, n_S, d_v] logits (fp32 values);
    rows: optional (b, i, s) triples.  Returns [B, T, n_S, d_v] or
    [n_rows, d_v]."""
    q, k, v = (_u16(a) for a in (q, k, v))
    B, T, n_H, d_qk = q.shape
    d_v = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != (B, T, n_H):
        raise ValueError("grouped shapes disagree")
    if group < 1 or n_H % (group + 1):
        raise ValueError("n_H must be a multiple of group + 1")
    n_S = group * (n_H // (group + 1))
    lam = np.ascontiguousarray(lam, dtype=np.float32).reshape(B, T, n_S)
    g = None if gate is None else np.ascontiguousarray(gate, dtype=np.float32).reshape(B, T, n_S, d_v)
    scale = 1.0 / np.sqrt(d_qk) if scale is None else float(scale)
    if rows is None:
        flat, n = None, B * T * n_S
    else:
        r = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
        flat = np.ascontiguousarray((r[:, 0] * T + r[:, 1]) * n_S + r[:, 2])
        n = flat.shape[0]
    out = np.empty((n, d_v), dtype=np.float64)
    rc = (lib or _load()).oracle_grouped(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, T, n_H, int(group), d_qk,
                                         d_v, lam.ctypes.data, None if g is None else g.ctypes.data, scale,
                                         None if flat is None else flat.ctypes.data, n, out.ctypes.data, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_grouped failed")
    return out.reshape(B, T, n_S, d_v) if rows is None else out
