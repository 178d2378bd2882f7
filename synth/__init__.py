"""Seeded synthetic inputs for causal differential attention.

This package only draws random numbers (see ``gen.c`` for the generator's
definition: counter-based SplitMix64, Box-Muller, one rounding to bf16).  It
holds none of the attention arithmetic; the HIP path's tests, the benchmark and
the fp64 oracle all take their inputs from here.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .workloads import WORKLOADS, Workload, TENSOR_IDS  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build() -> str:
    """Compile ``gen.c`` into ``libsynth.so`` beside it (gcc, OpenMP)."""
    import subprocess

    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", _LIB_PATH,
           os.path.join(_HERE, "gen.c"), "-lm"]
    subprocess.check_call(cmd)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, u32, i64 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64
        lib.synth_splitmix64.restype = u64
        lib.synth_splitmix64.argtypes = [u64, u64]
        lib.synth_stream_key.restype = u64
        lib.synth_stream_key.argtypes = [u64, u32]
        lib.synth_f64_to_bf16.restype = ctypes.c_uint16
        lib.synth_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.synth_normal_f64.argtypes = [u64, u32, u64, i64, ctypes.c_void_p]
        lib.synth_normal_bf16.argtypes = [u64, u32, u64, i64, ctypes.c_void_p]
        lib.synth_normal_f32.argtypes = [u64, u32, u64, i64, ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        lib.synth_uniform_f32.argtypes = [u64, u32, u64, i64, ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        _lib = lib
    return _lib


def splitmix64(x: int, k: int) -> int:
    """k-th output (0-based) of SplitMix64 seeded with x."""
    return int(_load().synth_splitmix64(x, k))


def f64_to_bf16(x: float) -> int:
    return int(_load().synth_f64_to_bf16(x))


def normal_f64(seed: int, tensor_id: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_normal_f64(seed, tensor_id, first, n, out.ctypes.data)
    return out


def normal_bf16(seed: int, tensor_id: int, shape, first: int = 0) -> np.ndarray:
    """bf16 N(0,1) entries as uint16 bit patterns, C-contiguous ``shape``."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    _load().synth_normal_bf16(seed, tensor_id, first, n, out.ctypes.data)
    return out.reshape(shape)


def normal_f32(seed: int, tensor_id: int, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_f32(seed, tensor_id, 0, n, mean, std, out.ctypes.data)
    return out.reshape(shape)


def uniform_f32(seed: int, tensor_id: int, shape, lo: float, hi: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    _load().synth_uniform_f32(seed, tensor_id, 0, n, lo, hi, out.ctypes.data)
    return out.reshape(shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def make_prefill_inputs(wl: Workload, B=None, T=None, H=None, seed=None) -> dict:
    """All inputs of one prefill call, drawn from the workload's recipe.

    Q1, Q2, K1, K2: bf16 [B, T, H, d_qk]; V: bf16 [B, T, H, d_v] (uint16 bits).
    gain: fp32 [H, d_v] = 1 + 0.02 N(0,1).  lam: fp32 [H] (scalar workloads
    repeat their lambda).  Sizes default to the workload's own.
    """
    B = wl.B if B is None else B
    T = wl.T if T is None else T
    H = wl.H if H is None else H
    seed = wl.seed if seed is None else seed
    ids = TENSOR_IDS
    x = {
        "q1": normal_bf16(seed, ids["q1"], (B, T, H, wl.d_qk)),
        "q2": normal_bf16(seed, ids["q2"], (B, T, H, wl.d_qk)),
        "k1": normal_bf16(seed, ids["k1"], (B, T, H, wl.d_qk)),
        "k2": normal_bf16(seed, ids["k2"], (B, T, H, wl.d_qk)),
        "v": normal_bf16(seed, ids["v"], (B, T, H, wl.d_v)),
        "gain": normal_f32(seed, ids["gain"], (H, wl.d_v), 1.0, 0.02),
        "lam": lambdas(wl, H, seed),
        "eps": wl.eps,
        "scale": wl.scale,
    }
    return x


def make_decode_inputs(wl: Workload, B=None, L=None, H=None, seed=None) -> dict:
    """Inputs of one decode call: q1, q2 bf16 [B, H, d_qk]; caches K1, K2
    bf16 [B, L, H, d_qk] and V bf16 [B, L, H, d_v]; gain, lam as for prefill."""
    B = wl.B if B is None else B
    L = wl.T if L is None else L
    H = wl.H if H is None else H
    seed = wl.seed if seed is None else seed
    ids = TENSOR_IDS
    return {
        "q1": normal_bf16(seed, ids["q1"], (B, H, wl.d_qk)),
        "q2": normal_bf16(seed, ids["q2"], (B, H, wl.d_qk)),
        "k1": normal_bf16(seed, ids["k1"], (B, L, H, wl.d_qk)),
        "k2": normal_bf16(seed, ids["k2"], (B, L, H, wl.d_qk)),
        "v": normal_bf16(seed, ids["v"], (B, L, H, wl.d_v)),
        "gain": normal_f32(seed, ids["gain"], (H, wl.d_v), 1.0, 0.02),
        "lam": lambdas(wl, H, seed),
        "eps": wl.eps,
        "scale": wl.scale,
    }


def lambdas(wl: Workload, H: int, seed: int) -> np.ndarray:
    if wl.lam_range is not None:
        lo, hi = wl.lam_range
        return uniform_f32(seed, TENSOR_IDS["lam"], (H,), lo, hi)
    return np.full((H,), wl.lam, dtype=np.float32)
