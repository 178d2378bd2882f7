"""GPU parity of grouped differential attention with token-wise lambda and
output gate (picx.dev summary of the Motif 3 report, section 2.2) through the
C ABI against the fp64 oracle.

Bounds: relative Frobenius error <= 5e-3 over the output (there is no
GroupNorm, so the output plays the role of the forward's pre-norm output and
takes its bound), and element by element
    |out - ref| <= 2e-2 * RMS_c(ref row)  [+ 2^-8 |ref| for bf16 output].
Rows differ in scale by orders of magnitude (an early row averages few values,
a late one thousands), so the element bound is relative to the row: the
computation's error is a few 1e-4 of the row's RMS (fp16 P and V, fp32
accumulation), and a lost or misplaced key tile moves the rows it touches by
far more.  The bf16 output mode adds its own rounding, at most 2^-9 of the
element (the gate makes a row's elements range widely, so this allowance is
per element, with a factor of 2 for the error the value had before rounding).
Every case prints its name first."""
import numpy as np
import pytest

import oracle
import synth
from tests.parity_util import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import differential_attention_causal_amd as da  # noqa: E402

REL = 5e-3
ELEM = 2e-2


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(B, T, n_H, g, seed, gate=True):
    n_S = g * (n_H // (g + 1))
    x = {"q": synth.normal_bf16(seed, 1, (B, T, n_H, 64)), "k": synth.normal_bf16(seed, 3, (B, T, n_H, 64)),
         "v": synth.normal_bf16(seed, 5, (B, T, n_H, 128)),
         "lam": synth.uniform_f32(seed, 7, (B, T, n_S), 0.0, 1.0)}
    # gate logits: bf16 N(0, 2^2) (tensor id 8), passed to the oracle as the same bf16 values
    x["gate"] = synth.f32_to_bf16_bits(synth.normal_f32(seed, 8, (B, T, n_S, 128), std=2.0)) if gate else None
    return x


def _gpu(x, g, out_dtype=torch.float32):
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    lam = torch.from_numpy(x["lam"]).cuda()
    gate = None if x["gate"] is None else to_dev(x["gate"])
    out = da.diffattn_fwd_grouped(q, k, v, g, lam, gate=gate, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _ref(x, g, rows=None):
    gate = None if x["gate"] is None else synth.bf16_bits_to_f32(x["gate"])
    return oracle.grouped(x["q"], x["k"], x["v"], g, x["lam"], gate=gate, rows=rows)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _elem(a, b, bf16):
    """Largest over elements of |a - b| / allowance, with the allowance
    ELEM * RMS of b's row (the last axis) [+ 2^-8 |b| for bf16 output]."""
    rms = np.sqrt(np.mean(b ** 2, axis=-1, keepdims=True))
    allow = ELEM * rms + (2.0 ** -8 * np.abs(b) if bf16 else 0.0)
    return float((np.abs(a - b) / np.maximum(allow, 1e-30)).max())


def _assert_close(got, ref, what, bf16=False):
    rel, elem = _rel(got, ref), _elem(got, ref, bf16)
    _say(what, "rel", rel, "err/allowance", elem)
    assert rel <= REL, (what, rel)
    assert elem <= 1.0, (what, elem)


@pytest.mark.parametrize("B,T,n_H,g,gate", [(1, 1, 2, 1, True), (1, 77, 2, 1, False), (2, 130, 4, 1, True),
                                            (1, 300, 4, 3, True), (2, 515, 8, 3, True), (1, 257, 6, 2, False)])
def test_grouped_all_rows(B, T, n_H, g, gate):
    _say("grouped", B, T, n_H, g, gate)
    x = _inputs(B, T, n_H, g, seed=600 + T + g, gate=gate)
    ref = _ref(x, g)
    _assert_close(_gpu(x, g), ref, "fp32 out")
    _assert_close(_gpu(x, g, torch.bfloat16), ref, "bf16 out", bf16=True)


def test_grouped_motif3_shape_every_row():
    # 16 heads, g = 3 (4 noise, 12 signal heads), T = 4096: the benchmark's
    # grouped shape, every output row
    _say("grouped B=1 T=4096 n_H=16 g=3, every row")
    x = _inputs(1, 4096, 16, 3, seed=31)
    ref = _ref(x, 3)
    _assert_close(_gpu(x, 3), ref, "fp32 out")
    _assert_close(_gpu(x, 3, torch.bfloat16), ref, "bf16 out", bf16=True)


def test_grouped_large_grid_sampled():
    # B=4, T=1100, 16 heads: 9 query blocks x 64 (b, head) = 576 blocks, more
    # than two per CU: the persistent ping-pong kernel runs several rounds
    _say("grouped B=4 T=1100 n_H=16 g=3 (grid of several rounds)")
    x = _inputs(4, 1100, 16, 3, seed=33)
    out = _gpu(x, 3)
    rng = np.random.default_rng(4)
    rows = sorted({(int(b), int(i), int(s)) for b, i, s in zip(rng.integers(0, 4, 60), rng.integers(0, 1100, 60),
                                                                rng.integers(0, 12, 60))}
                  | {(0, 0, 0), (3, 1099, 11), (1, 1023, 5), (2, 1024, 6)})
    ref = _ref(x, 3, rows=rows)
    got = np.stack([out[b, i, s] for b, i, s in rows])
    _assert_close(got, ref, "sampled")


def test_grouped_structure():
    _say("grouped: noise head feeds its g signal heads only; deterministic")
    x = _inputs(1, 200, 8, 3, seed=32)
    a = _gpu(x, 3)
    x2 = dict(x, v=x["v"].copy())
    x2["v"][:, :, 7] = synth.normal_bf16(998, 5, x2["v"][:, :, 7].shape)
    b = _gpu(x2, 3)
    assert np.array_equal(a[:, :, :3], b[:, :, :3])
    assert np.abs(a[:, :, 3:] - b[:, :, 3:]).max() > 1e-3
    assert np.array_equal(a, _gpu(x, 3))


@pytest.mark.parametrize("T,n_H", [(300, 8), (200, 260)])
def test_grouped_wide_key_stride(T, n_H):
    """A key row stride of 2^21 elements puts a head's key span past 2^31
    bytes: the ping-pong kernel's 32-bit offsets do not reach, and the
    register-staged kernels run instead (T=300, 8 heads: the two-group form;
    T=200, 260 heads: 520 blocks, more than two per CU, the four-wave form).
    Every output row against the oracle."""
    _say("grouped wide key stride", T, n_H)
    g = 3
    x = _inputs(1, T, n_H, g, seed=700 + n_H)
    st = 1 << 21
    base = torch.empty((T - 1) * st + n_H * 64, dtype=torch.bfloat16, device="cuda")
    k = base.as_strided((1, T, n_H, 64), (T * st, st, 64, 1))
    k.copy_(to_dev(x["k"]))
    q, v = to_dev(x["q"]), to_dev(x["v"])
    lam = torch.from_numpy(x["lam"]).cuda()
    gate = to_dev(x["gate"])
    out = da.diffattn_fwd_grouped(q, k, v, g, lam, gate=gate, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _assert_close(out.cpu().numpy(), _ref(x, g), "fp32 out")
    del base, k


@pytest.mark.parametrize("B,T,n_H", [(1, 8192, 8), (8, 1000, 16), (2, 4096, 16)])
def test_grouped_vt_tiles_every_row(B, T, n_H):
    """Shapes that take the V^T form on a 256-CU chip (V converted once into
    fp16 V^T tiles, moved by DMA): a one-round grid of a long sequence
    (T=8192), and two full rounds of pairs with a ragged last key tile
    (T=1000) or a whole one (T=4096).  Every output row against the oracle."""
    _say("grouped V^T form", B, T, n_H)
    x = _inputs(B, T, n_H, 3, seed=800 + T + n_H)
    ref = _ref(x, 3)
    _assert_close(_gpu(x, 3), ref, "fp32 out")
    _assert_close(_gpu(x, 3, torch.bfloat16), ref, "bf16 out", bf16=True)
