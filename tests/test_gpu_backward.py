"""GPU parity of the backward pass (diffattn_fwd_prefill_train +
diffattn_bwd_prefill, through the C ABI) against the fp64 autograd oracle
(oracle/backward.py).

Bound: every gradient tensor within 5e-3 relative Frobenius error of the
oracle's.  The kernels see exact bf16 inputs; the rounding they add is fp16
(2^-11 relative) on dO, P, dS and the transposed operands, plus fp32
accumulation, so the expected error is a few 1e-4; 5e-3 is the forward's
pre-norm bound, kept for the gradients.  Every case prints its name first."""
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
NAMES = ("dq1", "dq2", "dk1", "dk2", "dv", "dlam", "dgain")


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(B, T, H, seed, lam_range=(0.2, 0.9)):
    wl = Workload("bwd", "prefill", B=B, T=T, H=H, seed=seed, lam_range=lam_range)
    x = synth.make_prefill_inputs(wl)
    x["dy"] = synth.normal_bf16(seed, 9, (B, T, H, 128))  # dy: tensor id 9
    return x


def _gpu(x, dy_f32=False):
    q1, q2, k1, k2, v = (to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v"))
    gain, lam = f32_dev(x["gain"]), f32_dev(x["lam"])
    out, o1, o2, lse = da.diffattn_fwd_prefill_train(q1, q2, k1, k2, v, lam, gain, eps=x["eps"], scale=x["scale"])
    dy = to_dev(x["dy"])
    if dy_f32:
        dy = dy.float()
    g = da.diffattn_bwd_prefill(q1, q2, k1, k2, v, lam, gain, o1, o2, lse, dy, eps=x["eps"], scale=x["scale"])
    torch.cuda.synchronize()
    return {n: g[n].cpu().numpy().astype(np.float64) for n in NAMES}, (out, o1, o2, lse)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def _check(x, g, what):
    ref = bwd.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"], x["scale"],
                       synth.bf16_bits_to_f32(x["dy"]).astype(np.float64))
    rel = {n: _rel(g[n], ref[n]) for n in NAMES}
    _say("rel", {n: float("%.3g" % r) for n, r in rel.items()})
    for n in NAMES:
        assert np.isfinite(g[n]).all(), (what, n)
        if np.linalg.norm(ref[n]) <= 1e-9 * np.sqrt(ref[n].size):
            # the gradient vanishes (a softmax over one key has none): only
            # rounding may remain
            assert np.abs(g[n]).max() <= 1e-4, (what, n, np.abs(g[n]).max())
            continue
        assert rel[n] <= REL, (what, n, rel[n])


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
