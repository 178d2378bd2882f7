"""The prefill's workspace path (diffattn_fwd_prefill_ws without rope: V
converted once into fp16 V^T tiles that the kernels move by DMA) against the
plain entry point, through the C ABI.  On grids that fit the chip in one
round both run the ping-pong kernel, the same products on the same fp16
operands in the same order, so their outputs must agree bit for bit: small
and ragged lengths that leave part of the last V^T tile past T, a sliding
window wider than the streaming kernel takes, per-head lambda, a fused
strided layout.  On larger grids whose long/short pairs fill their rounds of
the chip (B=8 and T=16384 at 16 heads) the workspace path keeps the
persistent ping-pong kernel while the plain path runs the four-wave kernel:
two wave groups with their own reference maxima round P differently, so
there the two are held to the oracle's bounds and to each other within the
fp16 rounding of P.  Other larger grids (B=1, T=2048, 40 heads: 320 pairs on
256 CUs) run the four-wave kernel on both paths, with V^T tiles on the
workspace path.  The full-size workloads are also checked against the
oracle on sampled rows.  Every case prints its name first."""
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


def _dev_inputs(x, strided=False):
    if strided:
        fused = np.concatenate([x["q1"], x["q2"], x["k1"], x["k2"], x["v"]], axis=3)
        f = to_dev(fused)
        return f[..., 0:64], f[..., 64:128], f[..., 128:192], f[..., 192:256], f[..., 256:384]
    return tuple(to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v"))


def _same_kernel(B, T, H):
    """Both entry points run the ping-pong kernel: the grid of 128-query
    blocks fits the chip in one round (two blocks per CU)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return (T + 127) // 128 * B * H <= 2 * cus


def _agree(plain, pre_a, fast, pre_b, B, T, H):
    if _same_kernel(B, T, H):
        assert torch.equal(fast, plain) and torch.equal(pre_b, pre_a)
        return
    # different wave splits: the pre-norm outputs differ by the fp16 rounding
    # of P (relative 2^-11 per probability), averaged over the keys
    d = float(torch.linalg.vector_norm(pre_b - pre_a) / torch.linalg.vector_norm(pre_a))
    _say("workspace vs plain (different kernels): pre-norm rel-F %.3g" % d)
    assert d <= 1e-3


def _both(x, lam, window=0, strided=False, out_dtype=torch.float32):
    q1, q2, k1, k2, v = _dev_inputs(x, strided)
    gain = f32_dev(x["gain"])
    B, T, H, _ = x["q1"].shape
    pre_a = torch.empty((B, T, H, 128), dtype=torch.float32, device="cuda")
    pre_b = torch.empty_like(pre_a)
    plain = da.diffattn_fwd_prefill_ex(q1, q2, k1, k2, v, lam, gain, eps=x["eps"], scale=x["scale"],
                                       out_dtype=out_dtype, o_pre=pre_a, window=window)
    need = da.diffattn_prefill_workspace_bytes(B, T, H)
    assert need == B * H * ((T + 31) // 32) * 8192
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")  # contents need no initialisation
    fast = da.diffattn_fwd_prefill_ws(q1, q2, k1, k2, v, lam, gain, ws, eps=x["eps"], scale=x["scale"],
                                      out_dtype=out_dtype, o_pre=pre_b, window=window)
    torch.cuda.synchronize()
    return plain, pre_a, fast, pre_b


@pytest.mark.parametrize("B,T,H,window", [(1, 1, 1, 0), (1, 31, 2, 0), (1, 33, 2, 0), (2, 100, 3, 0),
                                          (1, 128, 2, 0), (1, 129, 2, 0), (3, 515, 4, 0), (1, 1000, 2, 0),
                                          (1, 4096, 2, 1000), (1, 2048, 40, 0), (2, 1100, 24, 300)])
def test_vtiles_bitwise_equal_plain(B, T, H, window):
    _say("V^T tiles vs plain", B, T, H, "window", window)
    wl = Workload("vt", "prefill", B=B, T=T, H=H, seed=300 + T, lam_range=(0.2, 0.9))
    x = synth.make_prefill_inputs(wl)
    lam = f32_dev(x["lam"])
    plain, pre_a, fast, pre_b = _both(x, lam, window=window)
    _agree(plain, pre_a, fast, pre_b, B, T, H)
    if T <= 1100 or not _same_kernel(B, T, H):
        o_ref, y_ref = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"],
                                      x["scale"], window=window)
        assert_parity(metrics(fast.cpu().numpy(), y_ref, pre_b.cpu().numpy(), o_ref), (B, T, H, window))


def test_vtiles_strided_layout_and_bf16_out():
    _say("V^T tiles: fused strided layout, bf16 output")
    wl = Workload("vts", "prefill", B=2, T=300, H=4, seed=31, lam=0.7)
    x = synth.make_prefill_inputs(wl)
    plain, pre_a, fast, pre_b = _both(x, 0.7, strided=True, out_dtype=torch.bfloat16)
    assert torch.equal(fast, plain) and torch.equal(pre_b, pre_a)


@pytest.mark.parametrize("name", ["prefill_b1_t4096_h16", "batch_b8_t4096_h16", "longctx_b1_t16384_h16"])
def test_vtiles_workloads(name):
    wl = synth.WORKLOADS[name]
    _say("V^T tiles, workload", name)
    x = synth.make_prefill_inputs(wl)
    lam = f32_dev(x["lam"]) if wl.lam_range is not None else wl.lam
    plain, pre_a, fast, pre_b = _both(x, lam, out_dtype=torch.bfloat16)
    _agree(plain, pre_a, fast, pre_b, wl.B, wl.T, wl.H)
    rng = np.random.default_rng(wl.seed)
    rows = sorted({(b, i, h) for b in {0, wl.B - 1} for h in {0, wl.H - 1} for i in (0, 31, 32, wl.T // 2, wl.T - 1)}
                  | {(int(rng.integers(wl.B)), int(rng.integers(wl.T)), int(rng.integers(wl.H))) for _ in range(24)})
    o_ref, y_ref = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"],
                                  x["scale"], rows=rows)
    idx = torch.tensor(rows, dtype=torch.long, device="cuda")
    m = metrics(fast[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy(), y_ref,
                pre_b[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy(), o_ref)
    _say("metrics", m)
    assert_parity(m, name)


def test_vtiles_workspace_refused_when_short():
    _say("V^T tiles: a short workspace is refused")
    wl = Workload("vtw", "prefill", B=1, T=100, H=2, seed=5)
    x = synth.make_prefill_inputs(wl)
    q1, q2, k1, k2, v = _dev_inputs(x)
    need = da.diffattn_prefill_workspace_bytes(1, 100, 2)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="workspace"):
        da.diffattn_fwd_prefill_ws(q1, q2, k1, k2, v, 0.8, f32_dev(x["gain"]), ws)


@pytest.mark.parametrize("B,T,H,window,rope", [(1, 300, 4, 0, da.ROPE_NONE), (2, 1000, 3, 0, da.ROPE_HALF),
                                               (1, 4096, 2, 1000, da.ROPE_NONE),
                                               (1, 129, 2, 300, da.ROPE_INTERLEAVED)])
def test_prepared_workspace(B, T, H, window, rope):
    """diffattn_prefill_prepare then diffattn_fwd_prefill_ws with the prepared
    flag equals the unprepared call bit for bit, and one preparation serves
    several calls with other queries over the same keys and values."""
    _say("prepared workspace", B, T, H, "window", window, "rope", rope)
    wl = Workload("vtp", "prefill", B=B, T=T, H=H, seed=700 + T + rope, lam=0.6)
    x = synth.make_prefill_inputs(wl)
    q1, q2, k1, k2, v = _dev_inputs(x)
    gain = f32_dev(x["gain"])
    kw = dict(eps=x["eps"], scale=x["scale"], out_dtype=torch.float32, window=window, rope=rope,
              rope_theta=5e5 if rope else 0.0, rope_pos0=3 if rope else 0)
    need = da.diffattn_prefill_workspace_bytes(B, T, H, rope=rope)
    ref_ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    da.diffattn_prefill_prepare(k1, k2, v, ws, window=window, rope=rope, rope_theta=kw["rope_theta"],
                                rope_pos0=kw["rope_pos0"])
    for qa, qb in ((q1, q2), (q2, q1), (q1, q1)):
        pre_a = torch.empty((B, T, H, 128), dtype=torch.float32, device="cuda")
        pre_b = torch.empty_like(pre_a)
        ref = da.diffattn_fwd_prefill_ws(qa, qb, k1, k2, v, 0.6, gain, ref_ws, o_pre=pre_a, **kw)
        got = da.diffattn_fwd_prefill_ws(qa, qb, k1, k2, v, 0.6, gain, ws, o_pre=pre_b, prepared=True, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got, ref) and torch.equal(pre_b, pre_a)
