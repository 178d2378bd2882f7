"""The five synthetic workloads, shaped like Motif 2.6B's attention layers.

Motif 2.6B (technical report, explained on the Motif 2.6B pages, section "The
block"): 16 heads with 16 KV heads, hidden size 2048; context 4,096 for the base
model and 16,384 for the long-context variant.  Differential attention splits a
head's query/key into two 64-wide halves (Q1/Q2, K1/K2) and keeps one 128-wide
value, so d_qk = 64 and d_v = 128.  Every entry is bf16 N(0,1); the GroupNorm
gain is 1 + 0.02 N(0,1) in fp32 and eps = 1e-5 (held as the fp32 value).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

TENSOR_IDS = {"q1": 1, "q2": 2, "k1": 3, "k2": 4, "v": 5, "gain": 6, "lam": 7}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    B: int
    T: int               # sequence length (prefill) or cache length L (decode)
    H: int
    seed: int
    lam: float = 0.8
    lam_range: Optional[Tuple[float, float]] = None  # per-head U(lo, hi) when set
    d_qk: int = 64
    d_v: int = 128
    num_splits: int = 0  # decode only
    eps: float = float(np.float32(1e-5))
    window: int = 0      # > 0: sliding window of that many keys (Motif 3's sliding-window layers)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    @property
    def causal_pairs(self) -> int:
        """(query, visible key) pairs over all rows and heads."""
        W = self.window if self.window > 0 else self.T
        if self.kind == "prefill":
            if W >= self.T:
                return self.B * self.H * self.T * (self.T + 1) // 2
            return self.B * self.H * (W * (W + 1) // 2 + (self.T - W) * W)
        return self.B * self.H * min(self.T, W)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_b1_h2_t128", "prefill", B=1, T=128, H=2, seed=1, lam=0.5),
        Workload("prefill_b1_t4096_h16", "prefill", B=1, T=4096, H=16, seed=2, lam=0.8),
        Workload("batch_b8_t4096_h16", "prefill", B=8, T=4096, H=16, seed=3, lam_range=(0.2, 0.9)),
        Workload("longctx_b1_t16384_h16", "prefill", B=1, T=16384, H=16, seed=4, lam=0.8),
        Workload("decode_b64_l4096_h16", "decode", B=64, T=4096, H=16, seed=5, lam=0.8, num_splits=8),
        # Sliding-window layers: 128-token windows are the window size the
        # picx.dev summary of the Motif 3 report quotes (section "Practical Implications").
        Workload("swa_b1_t16384_h16_w128", "prefill", B=1, T=16384, H=16, seed=6, lam=0.8, window=128),
        Workload("swa_decode_b64_l4096_h16_w128", "decode", B=64, T=4096, H=16, seed=7, lam=0.8,
                 num_splits=1, window=128),
    ]
}
