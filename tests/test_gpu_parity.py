"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small and ragged sizes compare every output element; the full-size workloads
compare sampled rows that the oracle computes one by one, in the same launch
configuration the benchmark times.  Every case prints its name first so a
failure is attributable.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.workloads import Workload
from tests.parity_util import assert_parity, f32_dev, metrics, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import differential_attention_causal_amd as da  # noqa: E402


def _say(*a):
    print("[case]", *a, flush=True)


def _prefill_gpu(x, out_dtype=torch.bfloat16, per_head=False, strided=False):
    dev = "cuda"
    if strided:
        # Q1, Q2, K1, K2, V as slices of one fused [B, T, H, 384] projection output.
        B, T, H, _ = x["q1"].shape
        fused = np.concatenate([x["q1"], x["q2"], x["k1"], x["k2"], x["v"]], axis=3)
        f = to_dev(fused, dev)
        q1, q2, k1, k2, v = f[..., 0:64], f[..., 64:128], f[..., 128:192], f[..., 192:256], f[..., 256:384]
    else:
        q1, q2, k1, k2, v = (to_dev(x[n], dev) for n in ("q1", "q2", "k1", "k2", "v"))
    gain = f32_dev(x["gain"], dev)
    lam = f32_dev(x["lam"], dev) if per_head else float(x["lam"][0])
    B, T, H, _ = x["q1"].shape
    o_pre = torch.empty((B, T, H, 128), dtype=torch.float32, device=dev)
    out = da.diffattn_fwd_prefill(q1, q2, k1, k2, v, lam, gain, eps=x["eps"], scale=x["scale"],
                                  out_dtype=out_dtype, o_pre=o_pre)
    torch.cuda.synchronize()
    return out, o_pre


def _inputs(B, T, H, seed, lam=0.8, lam_range=None):
    wl = Workload("case", "prefill", B=B, T=T, H=H, seed=seed, lam=lam, lam_range=lam_range)
    return synth.make_prefill_inputs(wl)


SMALL = [
    (1, 1, 1, 0.8), (1, 5, 2, 0.5), (1, 31, 1, 0.8), (1, 32, 2, 0.8), (1, 33, 2, 0.3), (2, 100, 3, 0.9),
    (1, 127, 2, 0.8), (1, 128, 2, 0.5), (1, 129, 2, 0.8), (2, 200, 2, -0.4), (1, 333, 3, 0.8),
    (1, 1000, 2, 0.8), (3, 515, 4, 0.95),
]


@pytest.mark.parametrize("B,T,H,lam", SMALL)
def test_prefill_small_all_rows(B, T, H, lam):
    _say("prefill all rows", B, T, H, lam)
    x = _inputs(B, T, H, seed=100 + T, lam=lam)
    o_ref, y_ref = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"],
                                  x["eps"], x["scale"])
    out, o_pre = _prefill_gpu(x)
    m = metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref)
    _say("metrics", m)
    assert_parity(m, (B, T, H, lam))
    out32, _ = _prefill_gpu(x, out_dtype=torch.float32)
    m32 = metrics(out32.cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref)
    assert_parity(m32, ("fp32 out", B, T, H, lam))


def test_prefill_per_head_lambda_and_strided_layout():
    _say("per-head lambda, fused strided layout")
    x = _inputs(2, 300, 4, seed=7, lam_range=(0.2, 0.9))
    o_ref, y_ref = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"],
                                  x["eps"], x["scale"])
    out, o_pre = _prefill_gpu(x, per_head=True)
    assert_parity(metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref), "per-head")
    out_s, o_pre_s = _prefill_gpu(x, per_head=True, strided=True)
    assert torch.equal(out_s, out) and torch.equal(o_pre_s, o_pre)


def _sample_rows(B, T, H, rng, n_random=24):
    rows = set()
    for b in {0, B - 1}:
        for h in {0, H - 1}:
            for i in (0, 1, 31, 32, 127, 128, 129, T // 2, T - 129, T - 2, T - 1):
                if 0 <= i < T:
                    rows.add((b, i, h))
    for _ in range(n_random):
        rows.add((int(rng.integers(B)), int(rng.integers(T)), int(rng.integers(H))))
    return sorted(rows)


@pytest.mark.parametrize("name", ["tiny_b1_h2_t128", "prefill_b1_t4096_h16", "batch_b8_t4096_h16",
                                  "longctx_b1_t16384_h16"])
def test_prefill_workloads(name):
    wl = synth.WORKLOADS[name]
    _say("workload", name)
    x = synth.make_prefill_inputs(wl)
    per_head = wl.lam_range is not None
    out, o_pre = _prefill_gpu(x, per_head=per_head)
    assert bool(torch.isfinite(out.float()).all())
    if name.startswith("tiny"):
        o_ref, y_ref = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"],
                                      x["eps"], x["scale"])
        m = metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref)
    else:
        rows = _sample_rows(wl.B, wl.T, wl.H, np.random.default_rng(wl.seed))
        o_ref, y_ref = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"],
                                      x["eps"], x["scale"], rows=rows)
        idx = torch.tensor(rows, dtype=torch.long, device="cuda")
        y = out[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy()
        o = o_pre[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy()
        m = metrics(y, y_ref, o, o_ref)
    _say("metrics", m)
    assert_parity(m, name)


def test_prefill_invariants():
    _say("invariants: V=ones, identical maps, causality, determinism, overwrite")
    x = _inputs(1, 260, 2, seed=3)
    # V = ones: rows of P1 - lambda P2 sum to 1 - lambda
    xo = dict(x, v=np.full_like(x["v"], 0x3F80))
    _, o_pre = _prefill_gpu(xo)
    assert float((o_pre - 0.2).abs().max()) < 2e-3
    # identical maps at lambda = 1 cancel exactly
    xi = dict(x, q2=x["q1"], k2=x["k1"], lam=np.ones_like(x["lam"]))
    out, o_pre = _prefill_gpu(xi)
    assert bool((o_pre == 0).all()) and bool((out.float() == 0).all())
    # causality: changing K/V/Q after position `cut` leaves rows <= cut bitwise unchanged
    cut = 140
    out_a, pre_a = _prefill_gpu(x)
    xc = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
    for n in ("q1", "q2", "k1", "k2", "v"):
        xc[n][:, cut + 1:] = synth.normal_bf16(999, 1, xc[n][:, cut + 1:].shape)
    out_c, pre_c = _prefill_gpu(xc)
    assert torch.equal(out_a[:, : cut + 1], out_c[:, : cut + 1])
    assert torch.equal(pre_a[:, : cut + 1], pre_c[:, : cut + 1])
    # run-to-run determinism
    out_b, pre_b = _prefill_gpu(x)
    assert torch.equal(out_a, out_b) and torch.equal(pre_a, pre_b)
    # NaN-prefilled outputs are fully overwritten
    B, T, H, _ = x["q1"].shape
    out_n = torch.full((B, T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    pre_n = torch.full((B, T, H, 128), float("nan"), dtype=torch.float32, device="cuda")
    da.diffattn_fwd_prefill(*(to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v")), float(x["lam"][0]),
                            f32_dev(x["gain"]), eps=x["eps"], scale=x["scale"], out=out_n, o_pre=pre_n)
    torch.cuda.synchronize()
    assert torch.equal(out_n, out_a) and torch.equal(pre_n, pre_a)


# ----------------------------- decode ------------------------------------

def _decode_gpu(x, seqlens=None, splits=0, out_dtype=torch.bfloat16, per_head=False):
    q1, q2, k1, k2, v = (to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v"))
    gain = f32_dev(x["gain"])
    lam = f32_dev(x["lam"]) if per_head else float(x["lam"][0])
    B, H, _ = x["q1"].shape
    sl = None if seqlens is None else torch.from_numpy(np.asarray(seqlens, np.int32)).cuda()
    o_pre = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    out = da.diffattn_fwd_decode(q1, q2, k1, k2, v, lam, gain, eps=x["eps"], scale=x["scale"], seqlens=sl,
                                 num_splits=splits, out_dtype=out_dtype, o_pre=o_pre)
    torch.cuda.synchronize()
    return out, o_pre


def _dec_inputs(B, L, H, seed, lam=0.8, lam_range=None):
    wl = Workload("dcase", "decode", B=B, T=L, H=H, seed=seed, lam=lam, lam_range=lam_range)
    return synth.make_decode_inputs(wl)


@pytest.mark.parametrize("B,L,H,splits", [(1, 1, 1, 8), (2, 7, 2, 8), (4, 300, 3, 8), (3, 1000, 2, 1),
                                          (2, 4096, 2, 16), (2, 1500, 2, 3), (1, 70000, 1, 8)])
def test_decode_small(B, L, H, splits):
    _say("decode", B, L, H, splits)
    x = _dec_inputs(B, L, H, seed=200 + L)
    o_ref, y_ref = oracle.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"],
                                 x["eps"], x["scale"])
    out, o_pre = _decode_gpu(x, splits=splits)
    m = metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref)
    _say("metrics", m)
    assert_parity(m, (B, L, H, splits))


def test_decode_ragged_seqlens_and_splits():
    _say("decode ragged seqlens, split invariance, per-head lambda")
    B, L, H = 6, 777, 2
    x = _dec_inputs(B, L, H, seed=9, lam_range=(0.2, 0.9))
    seqlens = [777, 1, 0, 5, 400, 9999]
    o_ref, y_ref = oracle.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"],
                                 x["eps"], x["scale"], seqlens=seqlens)
    outs = []
    for s in (1, 2, 4, 8, 16):
        out, o_pre = _decode_gpu(x, seqlens=seqlens, splits=s, per_head=True)
        m = metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref)
        assert_parity(m, ("splits", s))
        assert bool((out[2] == 0).all()) and bool((o_pre[2] == 0).all())  # empty cache -> zeros
        outs.append(o_pre)
    for o in outs[1:]:
        assert float((o - outs[0]).abs().max()) < 1e-5


def test_decode_equals_last_prefill_row():
    _say("decode vs last prefill row")
    x = _inputs(2, 513, 2, seed=4)
    out_p, pre_p = _prefill_gpu(x)
    xd = dict(x, q1=np.ascontiguousarray(x["q1"][:, -1]), q2=np.ascontiguousarray(x["q2"][:, -1]))
    out_d, pre_d = _decode_gpu(xd)
    assert float((pre_d - pre_p[:, -1]).abs().max()) < 2e-3
    assert float((out_d.float() - out_p[:, -1].float()).abs().max()) < 3e-2


def test_decode_workload_all_rows():
    wl = synth.WORKLOADS["decode_b64_l4096_h16"]
    _say("workload", wl.name)
    x = synth.make_decode_inputs(wl)
    o_ref, y_ref = oracle.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"],
                                 x["eps"], x["scale"])
    out, o_pre = _decode_gpu(x, splits=wl.num_splits)
    m = metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref)
    _say("metrics", m)
    assert_parity(m, wl.name)
