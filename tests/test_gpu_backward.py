"""GPU parity of the backward pass (diffattn_fwd_prefill_train +
diffattn_bwd_prefill, through the C ABI) against the fp64 autograd oracle
(oracle/backward.py).

Bounds, for every gradient tensor g against the oracle's r:
  - relative Frobenius error |g - r| / |r| <= 5e-3 (the forward's pre-norm
    bound, kept for the gradients);
  - element-wise max |g - r| <= 2e-2 * RMS(r).
The kernels see exact bf16 inputs; the rounding they add is fp16 (2^-11
relative) on dO, P, dS and the transposed operands, plus fp32 accumulation, so
the per-element error is a few 1e-4 of RMS(r) (measured relative Frobenius
errors are about 3e-4), and the largest of up to 4M such errors stays within
about six of their standard deviations: 2e-2 leaves a margin of about ten.  A
key or query tile whose contribution is lost or misplaced changes the elements
it touches by at least about 1/sqrt(128) (one of at most 128 query tiles) of
their size, which the element-wise bound catches where the norm would not.
Every case prints its name first."""
import numpy as np
import pytest

import synth
from oracle import backward as bwd
from synth.workloads import Workload
from tests.parity_util import f32_dev, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import differential_attention_causal_amd as da  # noqa: E402

REL = 5e-3
ELEM = 2e-2
NAMES = ("dq1", "dq2", "dk1", "dk2", "dv", "dlam", "dgain")


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(B, T, H, seed, lam_range=(0.2, 0.9)):
    wl = Workload("bwd", "prefill", B=B, T=T, H=H, seed=seed, lam_range=lam_range)
    x = synth.make_prefill_inputs(wl)
    x["dy"] = synth.normal_bf16(seed, 9, (B, T, H, 128))  # dy: tensor id 9
    return x


def _gpu(x, dy_f32=False, **var):
    q1, q2, k1, k2, v = (to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v"))
    gain, lam = f32_dev(x["gain"]), f32_dev(x["lam"])
    out, o1, o2, lse = da.diffattn_fwd_prefill_train(q1, q2, k1, k2, v, lam, gain, eps=x["eps"], scale=x["scale"],
                                                     **var)
    dy = to_dev(x["dy"])
    if dy_f32:
        dy = dy.float()
    g = da.diffattn_bwd_prefill(q1, q2, k1, k2, v, lam, gain, o1, o2, lse, dy, eps=x["eps"], scale=x["scale"],
                                **var)
    torch.cuda.synchronize()
    return {n: g[n].cpu().numpy().astype(np.float64) for n in NAMES}, (out, o1, o2, lse)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def _check(x, g, what, **var):
    ref = bwd.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"], x["scale"],
                       synth.bf16_bits_to_f32(x["dy"]).astype(np.float64), **var)
    _compare(g, ref, what)


def _compare(g, ref, what, names=NAMES):
    rel = {n: _rel(g[n], ref[n]) for n in names}
    elem = {n: float(np.abs(g[n] - ref[n]).max() / max(np.sqrt(np.mean(ref[n] ** 2)), 1e-30)) for n in names}
    _say("rel", {n: float("%.3g" % r) for n, r in rel.items()})
    _say("max/rms", {n: float("%.3g" % r) for n, r in elem.items()})
    for n in names:
        assert np.isfinite(g[n]).all(), (what, n)
        if np.linalg.norm(ref[n]) <= 1e-9 * np.sqrt(ref[n].size):
            # the gradient vanishes (a softmax over one key has none): only
            # rounding may remain
            assert np.abs(g[n]).max() <= 1e-4, (what, n, np.abs(g[n]).max())
            continue
        assert rel[n] <= REL, (what, n, rel[n])
        assert elem[n] <= ELEM, (what, n, elem[n])


# ragged sizes over several 32-row tiles and 128-row workgroups
@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (1, 33, 2), (2, 100, 2), (1, 128, 1), (1, 257, 3), (2, 515, 2)])
def test_backward_small(B, T, H):
    _say("backward", B, T, H)
    x = _inputs(B, T, H, seed=500 + T)
    g, _ = _gpu(x)
    _check(x, g, (B, T, H))


def test_backward_fp32_dy_and_scalar_lambda():
    _say("backward fp32 dy, one lambda")
    x = _inputs(1, 200, 2, seed=21, lam_range=None)
    g, _ = _gpu(x, dy_f32=True)
    _check(x, g, "fp32 dy")


def test_backward_one_gpu_share_t4096():
    # the T=4096 layer on one GPU's two heads (16 heads over 8 GPUs)
    _say("backward B=1 T=4096 H=2")
    x = _inputs(1, 4096, 2, seed=22)
    g, _ = _gpu(x)
    _check(x, g, "t4096")


def test_backward_deterministic_and_training_outputs():
    _say("backward determinism; training forward equals the plain forward")
    x = _inputs(1, 300, 2, seed=23)
    g1, (out, o1, o2, lse) = _gpu(x)
    g2, _ = _gpu(x)
    for n in NAMES:
        assert np.array_equal(g1[n], g2[n]), n
    q1, q2, k1, k2, v = (to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v"))
    plain = da.diffattn_fwd_prefill(q1, q2, k1, k2, v, f32_dev(x["lam"]), f32_dev(x["gain"]), eps=x["eps"],
                                    scale=x["scale"])
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    lam = f32_dev(x["lam"])[None, None, :, None]
    ref = bwd.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"], x["scale"],
                       np.zeros((1, 300, 2, 128)))
    assert _rel((o1 - lam * o2).cpu().numpy(), ref["o"]) < 5e-3
    # lse: log2 sum_j 2^(c s_ij); the row max bounds it below, + log2(i+1) above
    assert bool(torch.isfinite(lse).all())


def test_training_forward_large_grid():
    """The training forward on a grid larger than two workgroups per CU (the
    four-wave kernel, whose epilogue writes the training outputs): y equals the
    plain forward bitwise, o1 - lambda o2 matches the oracle's pre-norm output
    on sampled rows, and every log-sum-exp is finite."""
    import oracle

    _say("training forward, large grid (B=1, T=2048, H=40)")
    x = _inputs(1, 2048, 40, seed=24)
    q1, q2, k1, k2, v = (to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v"))
    lam, gain = f32_dev(x["lam"]), f32_dev(x["gain"])
    out, o1, o2, lse = da.diffattn_fwd_prefill_train(q1, q2, k1, k2, v, lam, gain, eps=x["eps"], scale=x["scale"])
    plain = da.diffattn_fwd_prefill(q1, q2, k1, k2, v, lam, gain, eps=x["eps"], scale=x["scale"])
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    rng = np.random.default_rng(24)
    rows = sorted({(0, i, h) for i in (0, 1, 127, 128, 1023, 2046, 2047) for h in (0, 39)}
                  | {(0, int(rng.integers(2048)), int(rng.integers(40))) for _ in range(24)})
    o_ref, _ = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"], x["scale"],
                              rows=rows)
    idx = torch.tensor(rows, dtype=torch.long, device="cuda")
    o = (o1 - lam[None, None, :, None] * o2)[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy()
    assert _rel(o, o_ref) < 5e-3
    assert bool(torch.isfinite(lse).all())


def _heads_subset(x, bs, hs):
    """The inputs of batch rows bs and heads hs alone (heads and batch rows are
    independent, so the oracle on the subset gives those rows' gradients)."""
    sub = {}
    for n in ("q1", "q2", "k1", "k2", "v", "dy"):
        sub[n] = np.ascontiguousarray(x[n][bs][:, :, hs])
    sub["lam"] = np.ascontiguousarray(np.asarray(x["lam"])[hs])
    sub["gain"] = np.ascontiguousarray(np.asarray(x["gain"])[hs])
    sub["eps"], sub["scale"] = x["eps"], x["scale"]
    return sub


@pytest.mark.parametrize("B,seed", [(1, 41), (8, 42)])
def test_backward_full_layer_h16(B, seed):
    """The whole 16-head T=4096 layer (the benchmark's backward shape), and the
    training-shaped batch B=8 with lambda per head, run at full size on the
    GPU; the oracle checks batch rows {0, B-1} x heads {0, 15}.  dlam and dgain
    sum over every batch row, so they are compared at B=1 only; at B=8 the
    five attention gradients are."""
    _say("backward full layer", B, 4096, 16)
    x = _inputs(B, 4096, 16, seed=seed)
    g, _ = _gpu(x)
    bs = [0] if B == 1 else [0, B - 1]
    hs = [0, 15]
    sub = _heads_subset(x, bs, hs)
    ref = bwd.backward(sub["q1"], sub["q2"], sub["k1"], sub["k2"], sub["v"], sub["lam"], sub["gain"], sub["eps"],
                       sub["scale"], synth.bf16_bits_to_f32(sub["dy"]).astype(np.float64))
    gs = {n: np.ascontiguousarray(g[n][bs][:, :, hs]) for n in ("dq1", "dq2", "dk1", "dk2", "dv")}
    names = NAMES
    if B == 1:
        gs["dlam"], gs["dgain"] = g["dlam"][hs], g["dgain"][hs]
    else:
        names = ("dq1", "dq2", "dk1", "dk2", "dv")
    _compare(gs, ref, ("full layer", B), names)


# The variants (diffattn_fwd_prefill_train_ex + diffattn_bwd_prefill_ex): the
# rotary embedding with both pairings (Motif 2.6B explainer, "The block"), the
# sliding window (picx.dev summary of the Motif 3 report, section 2.1), both
# together; ragged lengths, windows narrower and wider than a tile, a last
# case at T=4096 with the 128-token window of the Motif 3 sliding layers.
VARIANTS = [
    (1, 100, 2, dict(rope=da.ROPE_HALF, rope_theta=1e4, rope_pos0=5)),
    (2, 300, 2, dict(rope=da.ROPE_INTERLEAVED, rope_theta=5e5)),
    (1, 515, 2, dict(window=64)),
    (1, 257, 2, dict(window=2)),
    (1, 700, 3, dict(window=200, rope=da.ROPE_HALF, rope_theta=1e4)),
    (2, 1000, 2, dict(window=33, rope=da.ROPE_INTERLEAVED, rope_theta=1e4, rope_pos0=100)),
    (1, 4096, 2, dict(window=128, rope=da.ROPE_HALF, rope_theta=5e5)),
]


@pytest.mark.parametrize("B,T,H,var", VARIANTS)
def test_backward_variants(B, T, H, var):
    _say("backward variant", B, T, H, var)
    x = _inputs(B, T, H, seed=900 + T + var.get("window", 0))
    g, _ = _gpu(x, **var)
    _check(x, g, (B, T, H, var), **var)


def test_backward_rope_window_wide_equals_causal():
    # a window covering every key is the causal backward, bit for bit
    _say("backward window >= T equals causal")
    x = _inputs(1, 300, 2, seed=31)
    g0, _ = _gpu(x, rope=da.ROPE_HALF, rope_theta=5e5)
    g1, _ = _gpu(x, rope=da.ROPE_HALF, rope_theta=5e5, window=300)
    for n in NAMES:
        assert np.array_equal(g0[n], g1[n]), n


def test_backward_single_key_window():
    """window = 1: every softmax covers one key (P = 1), so the exact dQ and
    dK vanish; what the kernels leave is the difference of two fp32
    evaluations of the same row dot product (D from the fp32 forward output,
    dP from the fp16 operands), a few 1e-4 of the gradients' natural scale,
    bounded here by 1e-3 of dV's RMS.  dV and dgain keep the usual bounds;
    dlambda, a sum over B*T*128 signed products that nearly cancel, is held
    to a relative 2e-2."""
    _say("backward window 1")
    x = _inputs(1, 257, 2, seed=1258)
    g, _ = _gpu(x, window=1)
    ref = bwd.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"], x["scale"],
                       synth.bf16_bits_to_f32(x["dy"]).astype(np.float64), window=1)
    _compare(g, ref, "window 1", names=("dv", "dgain"))
    scale = float(np.sqrt(np.mean(ref["dv"] ** 2)))
    for n in ("dq1", "dq2", "dk1", "dk2"):
        assert np.abs(ref[n]).max() <= 1e-12 * scale, n
        assert np.abs(g[n]).max() <= 1e-3 * scale, (n, np.abs(g[n]).max(), scale)
    assert _rel(g["dlam"], ref["dlam"]) <= 2e-2, (g["dlam"], ref["dlam"])
