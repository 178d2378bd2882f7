"""GPU parity of the rotary position embedding (Motif 2.6B explainer, section
"The block": RoPE with base 500,000) through the C ABI against the fp64
oracle: the standalone rotation, the prefill with its rotation of Q1, Q2, K1,
K2 (alone and with a sliding window) in both forms (keys rotated once into the
workspace by diffattn_fwd_prefill_ws, or inside the kernels by
diffattn_fwd_prefill_ex), and the decode, which rotates its query against a
cache of already rotated keys.  Every case prints its name first so a failure
is attributable."""
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

THETA = 500000.0


def _say(*a):
    print("[case]", *a, flush=True)


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _rot_bound(ref):
    # bf16 rounding of the rotated value (half an ulp, 2^-9 relative) plus the
    # angle's error (the fp32 phase and the hardware sine, well under 1e-5)
    return np.abs(ref) * 2.0 ** -8 + 2e-5


@pytest.mark.parametrize("mode", [1, 2])
def test_rope_apply(mode):
    _say("rope_apply", mode)
    x = synth.normal_bf16(71, 1, (3, 50, 4, 64))
    for pos0, ps in [(0, None), (1000, [0, 7, 123456]), ((1 << 30) + 5, [3, 0, 1])]:
        ref = oracle.rope(x, mode, THETA, pos0=pos0, pos_start=ps)
        xd = to_dev(x)
        psd = None if ps is None else torch.tensor(ps, dtype=torch.int32, device="cuda")
        out = da.diffattn_rope_apply(xd, mode, THETA, pos0=pos0, pos_start=psd)
        torch.cuda.synchronize()
        got = synth.bf16_bits_to_f32(_bits(out)).astype(np.float64)
        err = np.abs(got - ref)
        _say("pos0", pos0, "max err", float(err.max()))
        assert (err <= _rot_bound(ref)).all(), (pos0, float(err.max()))
        # in place gives the same bits
        da.diffattn_rope_apply(xd, mode, THETA, pos0=pos0, pos_start=psd, out=xd)
        torch.cuda.synchronize()
        assert torch.equal(xd, out)


def test_rope_apply_strided():
    _say("rope_apply strided in and out")
    x = synth.normal_bf16(72, 1, (2, 33, 3, 64))
    fused = torch.zeros((2, 33, 3, 192), dtype=torch.bfloat16, device="cuda")
    fused[..., 64:128] = to_dev(x)
    cache = torch.zeros((2, 40, 3, 128), dtype=torch.bfloat16, device="cuda")
    da.diffattn_rope_apply(fused[..., 64:128], 1, THETA, pos0=9, out=cache[:, :33, :, 64:])
    plain = da.diffattn_rope_apply(to_dev(x), 1, THETA, pos0=9)
    torch.cuda.synchronize()
    assert torch.equal(cache[:, :33, :, 64:], plain)
    assert bool((cache[:, 33:] == 0).all()) and bool((cache[..., :64] == 0).all())


def _inputs(B, T, H, seed, lam=0.8, lam_range=None):
    wl = Workload("case", "prefill", B=B, T=T, H=H, seed=seed, lam=lam, lam_range=lam_range)
    return synth.make_prefill_inputs(wl)


def _prefill(x, mode, pos0=0, window=0, per_head=False, ws=True):
    q1, q2, k1, k2, v = (to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v"))
    gain = f32_dev(x["gain"])
    lam = f32_dev(x["lam"]) if per_head else float(x["lam"][0])
    B, T, H, _ = x["q1"].shape
    o_pre = torch.empty((B, T, H, 128), dtype=torch.float32, device="cuda")
    out = da.diffattn_fwd_prefill_ex(q1, q2, k1, k2, v, lam, gain, eps=x["eps"], scale=x["scale"], o_pre=o_pre,
                                     window=window, rope=mode, rope_theta=THETA, rope_pos0=pos0, workspace=ws)
    torch.cuda.synchronize()
    return out, o_pre


# Small grids take the split-key workgroups (ping-pong with pre-rotated keys,
# lock-step with the rotation inside), the (1, 8192, 16) grid the four-wave
# one.
@pytest.mark.parametrize("ws", [True, False], ids=["keys-rotated-once", "rotated-in-kernel"])
@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B,T,H,pos0,window", [(1, 1, 1, 0, 0), (1, 77, 2, 0, 0), (2, 300, 3, 5, 0),
                                               (1, 515, 2, 100000, 0), (1, 700, 2, 3, 128)])
def test_prefill_rope_all_rows(mode, B, T, H, pos0, window, ws):
    _say("prefill rope all rows", mode, B, T, H, pos0, window, "workspace" if ws else "in-kernel")
    x = _inputs(B, T, H, seed=400 + T)
    o_ref, y_ref = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"],
                                  x["scale"], window=window, rope=mode, rope_theta=THETA, rope_pos0=pos0)
    out, o_pre = _prefill(x, mode, pos0=pos0, window=window, ws=ws)
    m = metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref)
    _say("metrics", m)
    assert_parity(m, (mode, B, T, H, pos0, window, ws))


@pytest.mark.parametrize("mode", [1, 2])
def test_prefill_rope_two_forms_agree(mode):
    # Both forms rotate the keys in fp32 and round them to fp16; the two code
    # paths may contract the rotation's products differently (a last-bit
    # difference in some rotated keys), and their kernels sum in different
    # orders: far below the 5e-3 parity bound, well above fp32 rounding.
    _say("prefill rope: workspace form vs in-kernel form", mode)
    x = _inputs(2, 333, 3, seed=77 + mode)
    _, a = _prefill(x, mode, pos0=11, ws=True)
    _, b = _prefill(x, mode, pos0=11, ws=False)
    rel = float((a - b).norm() / b.norm())
    _say("rel", rel)
    assert rel < 1e-4
    # a caller's workspace, reused by a second call of another size
    q = {n: to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v")}
    need = da.diffattn_prefill_workspace_bytes(2, 333, 3, rope=mode)
    wsbuf = torch.empty(need, dtype=torch.uint8, device="cuda")
    o1 = torch.empty((2, 333, 3, 128), dtype=torch.float32, device="cuda")
    da.diffattn_fwd_prefill_ws(q["q1"], q["q2"], q["k1"], q["k2"], q["v"], float(x["lam"][0]), f32_dev(x["gain"]),
                               wsbuf, eps=x["eps"], scale=x["scale"], o_pre=o1, rope=mode, rope_theta=THETA,
                               rope_pos0=11)
    y = _inputs(1, 100, 3, seed=5)
    _, c = _prefill(y, mode, pos0=11, ws=wsbuf)
    _, d = _prefill(y, mode, pos0=11, ws=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, a) and torch.equal(c, d)
    # rope on without a workspace is an error of the _ws entry point
    with pytest.raises(RuntimeError, match="workspace"):
        da.diffattn_fwd_prefill_ws(q["q1"], q["q2"], q["k1"], q["k2"], q["v"], 0.5, f32_dev(x["gain"]), None,
                                   rope=mode, rope_theta=THETA)


def _rows(B, T, H, rng, n_random=40):
    rows = {(b, i, h) for b in {0, B - 1} for h in {0, H - 1} for i in (0, 1, 127, 128, T // 2, T - 1)}
    for _ in range(n_random):
        rows.add((int(rng.integers(B)), int(rng.integers(T)), int(rng.integers(H))))
    return sorted(rows)


# (2, 1, 2048, 40, True): 320 long/short pairs on 256 CUs do not fill two
# rounds, so the workspace path runs the four-wave kernel with V^T tiles and
# pre-rotated keys; T=8192 at 16 heads fills two rounds (ping-pong kernel).
@pytest.mark.parametrize("mode,B,T,H,ws", [(1, 1, 4096, 16, True), (2, 1, 4096, 16, True), (1, 1, 8192, 16, True),
                                         (2, 1, 8192, 16, False), (2, 1, 2048, 40, True)])
def test_prefill_rope_large_sampled(mode, B, T, H, ws):
    _say("prefill rope sampled rows", mode, B, T, H, ws)
    x = _inputs(B, T, H, seed=T + mode)
    out, o_pre = _prefill(x, mode, ws=ws)
    assert bool(torch.isfinite(out.float()).all())
    rows = _rows(B, T, H, np.random.default_rng(T))
    o_ref, y_ref = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"],
                                  x["scale"], rows=rows, rope=mode, rope_theta=THETA)
    idx = torch.tensor(rows, dtype=torch.long, device="cuda")
    m = metrics(out[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy(), y_ref,
                o_pre[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy(), o_ref)
    _say("metrics", m)
    assert_parity(m, (mode, B, T, H))


# Windows of at most four key tiles before the diagonal one (W <= 129) with
# the keys rotated once take the streaming window kernel, which turns each
# block's queries itself; the in-kernel form keeps the plain kernels with
# tile skipping.
@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B,T,H,pos0,window,per_head", [(1, 33, 2, 0, 1, False), (2, 333, 3, 7, 32, True),
                                                        (1, 515, 2, 1000, 33, False), (1, 1000, 3, 3, 100, True),
                                                        (2, 640, 2, 0, 129, False)])
def test_prefill_rope_window_streaming(mode, B, T, H, pos0, window, per_head):
    _say("prefill rope window streaming kernel", mode, B, T, H, pos0, window, per_head)
    x = _inputs(B, T, H, seed=900 + T + window, lam_range=(0.2, 0.9) if per_head else None)
    o_ref, y_ref = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"],
                                  x["scale"], window=window, rope=mode, rope_theta=THETA, rope_pos0=pos0)
    out, o_pre = _prefill(x, mode, pos0=pos0, window=window, per_head=per_head, ws=True)
    m = metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref)
    _say("metrics", m)
    assert_parity(m, (mode, B, T, H, pos0, window))
    # the in-kernel rotation form (plain kernels, tiles outside the window
    # skipped) agrees well inside the 5e-3 parity bound: the two forms may
    # round a rotated key to fp16 differently in the last bit, and with a
    # short window each output sums few terms, so such a bit weighs more than
    # in the causal comparison above (measured 1.7e-4 at W = 32)
    _, o_in = _prefill(x, mode, pos0=pos0, window=window, per_head=per_head, ws=False)
    rel = float((o_pre - o_in).norm() / o_in.norm())
    _say("streaming vs in-kernel rel", rel)
    assert rel < 1e-3


@pytest.mark.parametrize("mode", [1, 2])
def test_prefill_rope_window_long_sampled(mode):
    # a Motif 3 sliding-window layer shape: 16 heads, 128-token window, long prompt
    B, T, H, W = 1, 16384, 16, 128
    _say("prefill rope window sampled rows", mode, B, T, H, W)
    x = _inputs(B, T, H, seed=31 + mode)
    out, o_pre = _prefill(x, mode, pos0=5, window=W, ws=True)
    assert bool(torch.isfinite(out.float()).all())
    rows = _rows(B, T, H, np.random.default_rng(T + mode))
    o_ref, y_ref = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"],
                                  x["scale"], rows=rows, window=W, rope=mode, rope_theta=THETA, rope_pos0=5)
    idx = torch.tensor(rows, dtype=torch.long, device="cuda")
    m = metrics(out[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy(), y_ref,
                o_pre[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy(), o_ref)
    _say("metrics", m)
    assert_parity(m, (mode, B, T, H, W))


@pytest.mark.parametrize("mode,B,T,H,pos0", [(1, 1, 100, 3, 0), (2, 2, 1000, 4, 17), (1, 1, 4096, 16, 0)])
def test_prepared_rope_workspace_contents(mode, B, T, H, pos0):
    """The pre-pass alone (diffattn_prefill_prepare with rope: the key
    rotation and the V^T tiles in one launch).  The rotated keys at the head
    of the workspace (fp16, C-contiguous, K1 then K2 at 256-byte aligned
    offsets) are held to the fp64 rotation within fp16 rounding; the V^T tiles
    after them equal, byte for byte, those that the preparation without rope
    writes (the two workspaces start from different fill bytes, so equal
    bytes mean both were written)."""
    _say("prepared rope workspace contents", mode, B, T, H, "pos0", pos0)
    wl = Workload("rws", "prefill", B=B, T=T, H=H, seed=900 + T + mode, lam=0.5)
    x = synth.make_prefill_inputs(wl)
    k1, k2, v = to_dev(x["k1"]), to_dev(x["k2"]), to_dev(x["v"])
    need_r = da.diffattn_prefill_workspace_bytes(B, T, H, rope=mode)
    need_p = da.diffattn_prefill_workspace_bytes(B, T, H)
    one = (B * T * H * 64 * 2 + 255) // 256 * 256
    assert need_r == 2 * one + need_p
    ws_r = torch.full((need_r,), 0x5A, dtype=torch.uint8, device="cuda")
    ws_p = torch.full((need_p,), 0xA5, dtype=torch.uint8, device="cuda")
    da.diffattn_prefill_prepare(k1, k2, v, ws_r, rope=mode, rope_theta=THETA, rope_pos0=pos0)
    da.diffattn_prefill_prepare(k1, k2, v, ws_p)
    torch.cuda.synchronize()
    assert torch.equal(ws_r[2 * one:], ws_p)
    n = B * T * H * 64
    for i, name in enumerate(("k1", "k2")):
        got = ws_r[i * one:i * one + 2 * n].view(torch.float16).float().cpu().numpy().astype(np.float64)
        ref = oracle.rope(x[name], mode, THETA, pos0=pos0).reshape(-1)
        err = np.abs(got - ref)
        _say(name, "max err", float(err.max()))
        # fp16 rounding (half an ulp, 2^-11 relative) plus the angle's error
        assert (err <= np.abs(ref) * 2.0 ** -10 + 2e-5).all(), (name, float(err.max()))


def test_prefill_rope_shift_invariance():
    _say("prefill rope: moving every token leaves the result (up to rounding)")
    x = _inputs(1, 400, 2, seed=9)
    _, a = _prefill(x, 1, pos0=0)
    _, b = _prefill(x, 1, pos0=1 << 20)
    rel = float((a - b).norm() / a.norm())
    _say("rel", rel)
    assert rel < 5e-3


def _dec_inputs(B, L, H, seed, lam=0.8):
    wl = Workload("dcase", "decode", B=B, T=L, H=H, seed=seed, lam=lam)
    return synth.make_decode_inputs(wl)


@pytest.mark.parametrize("mode", [1, 2])
def test_decode_rope(mode):
    _say("decode rope", mode)
    x = _dec_inputs(5, 900, 2, seed=80 + mode)
    seqlens = [900, 1, 0, 333, 5000]
    pos0 = 17
    o_ref, y_ref = oracle.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"],
                                 x["scale"], seqlens=seqlens, rope=mode, rope_theta=THETA, rope_pos0=pos0)
    q1, q2, k1, k2, v = (to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v"))
    sl = torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    for s in (1, 8):
        o_pre = torch.empty((5, 2, 128), dtype=torch.float32, device="cuda")
        out = da.diffattn_fwd_decode_ex(q1, q2, k1, k2, v, float(x["lam"][0]), f32_dev(x["gain"]), eps=x["eps"],
                                        scale=x["scale"], seqlens=sl, num_splits=s, o_pre=o_pre, rope=mode,
                                        rope_theta=THETA, rope_pos0=pos0)
        torch.cuda.synchronize()
        m = metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref)
        _say("splits", s, "metrics", m)
        assert_parity(m, ("decode rope", mode, s))


@pytest.mark.parametrize("mode", [1, 2])
def test_decode_with_rotated_cache_equals_last_prefill_row(mode):
    _say("decode on a cache from diffattn_rope_apply vs last prefill row", mode)
    x = _inputs(2, 513, 2, seed=15)
    _, pre_p = _prefill(x, mode, pos0=40)
    k1 = da.diffattn_rope_apply(to_dev(x["k1"]), mode, THETA, pos0=40)
    k2 = da.diffattn_rope_apply(to_dev(x["k2"]), mode, THETA, pos0=40)
    q1 = to_dev(np.ascontiguousarray(x["q1"][:, -1]))
    q2 = to_dev(np.ascontiguousarray(x["q2"][:, -1]))
    o_pre = torch.empty((2, 2, 128), dtype=torch.float32, device="cuda")
    da.diffattn_fwd_decode_ex(q1, q2, k1, k2, to_dev(x["v"]), float(x["lam"][0]), f32_dev(x["gain"]),
                              eps=x["eps"], scale=x["scale"], o_pre=o_pre, rope=mode, rope_theta=THETA, rope_pos0=40)
    torch.cuda.synchronize()
    # the cache holds bf16-rounded rotated keys, the prefill fp16-rounded ones
    rel = float((o_pre - pre_p[:, -1]).norm() / pre_p[:, -1].norm())
    _say("rel", rel)
    assert rel < 5e-3
