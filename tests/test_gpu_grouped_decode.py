"""GPU parity of the grouped differential-attention decode
(diffattn_fwd_grouped_decode: the newest token of each sequence against its
cache; picx.dev summary of the Motif 3 report, section 2.2) through the C ABI
against the fp64 oracle.  The oracle is the grouped prefill's definition
(oracle.grouped): a sequence's visible cache positions, in order, become a
prefill sequence whose last row holds the decode query (and its lambda and
gate), and that last row is the expected output; there is no position in the
operation but the order of the keys, so the two agree by definition.  Bounds
as for the grouped prefill (tests/test_gpu_grouped.py): relative Frobenius
5e-3 over the output, and element by element 2e-2 of the row's RMS [+ 2^-8 of
the element for bf16 output].  Every case prints its name first."""
import numpy as np
import pytest

import oracle
import synth
from tests.parity_util import to_dev
from tests.test_gpu_grouped import _assert_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import differential_attention_causal_amd as da  # noqa: E402


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(B, L, n_H, g, seed, gate=True):
    n_S = g * (n_H // (g + 1))
    x = {"q": synth.normal_bf16(seed, 1, (B, n_H, 64)), "k": synth.normal_bf16(seed, 3, (B, L, n_H, 64)),
         "v": synth.normal_bf16(seed, 5, (B, L, n_H, 128)),
         "lam": synth.uniform_f32(seed, 7, (B, n_S), 0.0, 1.0)}
    x["gate"] = synth.f32_to_bf16_bits(synth.normal_f32(seed, 8, (B, n_S, 128), std=2.0)) if gate else None
    return x


def _ref(x, g, seqlens, window=0, ring=False):
    """Expected [B, n_S, 128] from oracle.grouped, one sequence at a time."""
    B, L, n_H, _ = x["k"].shape
    n_S = g * (n_H // (g + 1))
    out = np.zeros((B, n_S, 128))
    for b in range(B):
        n = int(seqlens[b]) if seqlens is not None else L
        if not ring:
            n = min(n, L)
        lo = max(0, n - window) if window > 0 else (max(0, n - L) if ring else 0)
        if n - lo <= 0:
            continue
        slots = np.arange(lo, n) % L  # a linear cache has n <= L: slot = position
        m = n - lo
        q = np.zeros((1, m, n_H, 64), np.uint16)
        q[0, -1] = x["q"][b]
        lam = np.zeros((1, m, n_S), np.float32)
        lam[0, -1] = x["lam"][b]
        gate = None
        if x["gate"] is not None:
            gate = np.zeros((1, m, n_S, 128), np.float32)
            gate[0, -1] = synth.bf16_bits_to_f32(x["gate"][b])
        out[b] = oracle.grouped(q, x["k"][b:b + 1, slots], x["v"][b:b + 1, slots], g, lam, gate=gate,
                                rows=[(0, m - 1, s) for s in range(n_S)])
    return out


def _gpu(x, g, seqlens=None, out_dtype=torch.float32, **kw):
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    lam = torch.from_numpy(x["lam"]).cuda()
    gate = None if x["gate"] is None else to_dev(x["gate"])
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    out = da.diffattn_fwd_grouped_decode(q, k, v, g, lam, gate=gate, seqlens=sl, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


@pytest.mark.parametrize("B,L,n_H,g,gate,splits", [(1, 1, 2, 1, True, 1), (2, 77, 4, 1, False, 8),
                                                   (3, 600, 4, 3, True, 8), (2, 1000, 8, 3, True, 3),
                                                   (1, 2049, 6, 2, False, 64)])
def test_grouped_decode_all_lengths(B, L, n_H, g, gate, splits):
    _say("grouped decode", B, L, n_H, g, "gate", gate, "splits", splits)
    x = _inputs(B, L, n_H, g, seed=40 + L + n_H, gate=gate)
    rng = np.random.default_rng(L)
    seqlens = [L] + [int(rng.integers(1, L + 1)) for _ in range(B - 1)]
    got = _gpu(x, g, seqlens=seqlens, num_splits=splits)
    _assert_close(got, _ref(x, g, seqlens), (B, L, n_H, g, gate, splits))


def test_grouped_decode_ragged_empty_and_bf16():
    # lengths 0 (output 0), 1, past L (clamped to L for a linear cache)
    _say("grouped decode: ragged lengths, bf16 output")
    x = _inputs(4, 300, 4, 1, seed=55)
    seqlens = [0, 1, 299, 1000]
    got = _gpu(x, 1, seqlens=seqlens, out_dtype=torch.bfloat16)
    ref = _ref(x, 1, seqlens)
    assert np.all(got[0] == 0)
    _assert_close(got[1:], ref[1:], "ragged bf16", bf16=True)


@pytest.mark.parametrize("window,ring", [(64, False), (128, True), (0, True)])
def test_grouped_decode_window_and_ring(window, ring):
    _say("grouped decode window", window, "ring", ring)
    x = _inputs(3, 512, 4, 3, seed=60 + window)
    seqlens = [512, 700, 1500] if ring else [512, 100, 33]
    got = _gpu(x, 3, seqlens=seqlens, window=window, kv_ring=ring)
    _assert_close(got, _ref(x, 3, seqlens, window=window, ring=ring), ("window", window, "ring", ring))


def test_grouped_decode_motif3_shape():
    # the decode benchmark's shape: B=64 sequences of 4096 cached tokens, 16
    # heads (12 signal, 4 noise, g=3), token-wise lambda and gate; the oracle
    # on 6 of the 64 sequences
    _say("grouped decode B=64 L=4096 16 heads g=3")
    x = _inputs(64, 4096, 16, 3, seed=77)
    got = _gpu(x, 3)
    idx = [0, 1, 17, 40, 62, 63]
    sub = {n: (None if x[n] is None else x[n][idx]) for n in x}
    _assert_close(got[idx], _ref(sub, 3, None), "motif3 shape")
