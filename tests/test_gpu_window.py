"""GPU parity of the sliding-window variant (the sliding-window layers in the
picx.dev summary of the Motif 3 report, section 2.1): prefill with a window,
decode with a window over a linear cache, and decode over a ring-buffer cache,
each through the C ABI against the fp64 oracle.  Every case prints its name
first so a failure is attributable."""
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


def _inputs(B, T, H, seed, lam=0.8, lam_range=None):
    wl = Workload("case", "prefill", B=B, T=T, H=H, seed=seed, lam=lam, lam_range=lam_range)
    return synth.make_prefill_inputs(wl)


def _prefill(x, window, per_head=False, out_dtype=torch.bfloat16, ex=True):
    q1, q2, k1, k2, v = (to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v"))
    gain = f32_dev(x["gain"])
    lam = f32_dev(x["lam"]) if per_head else float(x["lam"][0])
    B, T, H, _ = x["q1"].shape
    o_pre = torch.empty((B, T, H, 128), dtype=torch.float32, device="cuda")
    if ex:
        out = da.diffattn_fwd_prefill_ex(q1, q2, k1, k2, v, lam, gain, eps=x["eps"], scale=x["scale"],
                                         out_dtype=out_dtype, o_pre=o_pre, window=window)
    else:
        out = da.diffattn_fwd_prefill(q1, q2, k1, k2, v, lam, gain, eps=x["eps"], scale=x["scale"],
                                      out_dtype=out_dtype, o_pre=o_pre)
    torch.cuda.synchronize()
    return out, o_pre


def _oracle_prefill(x, window, rows=None):
    return oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"], x["eps"],
                          x["scale"], rows=rows, window=window)


# Windows of at most four key tiles before the diagonal one (w <= 129) run the
# streaming kernel (four query blocks per workgroup, key tiles through a ring);
# deeper windows the split-key or four-wave kernels, which skip the tiles
# before each wave's window.  The cases span every depth 0..4 of the
# streaming kernel (w = 1, 7, 31, 32, 33; 64, 65; 96; 100, 128, 129), ragged
# ends, several blocks per workgroup and several workgroups per head.
SMALL = [
    (1, 64, 1, 31), (1, 129, 2, 33), (1, 333, 2, 1), (1, 333, 2, 7), (2, 200, 3, 32), (1, 515, 2, 100),
    (1, 1000, 2, 128), (1, 1000, 2, 129), (2, 700, 2, 1000), (1, 257, 2, 96), (1, 700, 2, 64), (2, 600, 3, 65),
]


@pytest.mark.parametrize("B,T,H,W", SMALL)
def test_prefill_window_all_rows(B, T, H, W):
    _say("prefill window all rows", B, T, H, W)
    x = _inputs(B, T, H, seed=300 + T + W)
    o_ref, y_ref = _oracle_prefill(x, W)
    out, o_pre = _prefill(x, W)
    m = metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref)
    _say("metrics", m)
    assert_parity(m, (B, T, H, W))


@pytest.mark.parametrize("W", [100, 128])
def test_prefill_window_options(W):
    """The streaming kernel with per-head lambda, fp32 output, no pre-norm
    output, and Q1, Q2, K1, K2, V as slices of one fused [B, T, H, 384]
    projection output (row strides of 384 elements)."""
    _say("prefill window options", W)
    B, T, H = 2, 450, 3
    x = _inputs(B, T, H, seed=500 + W, lam_range=(0.2, 0.9))
    o_ref, y_ref = _oracle_prefill(x, W)
    out, o_pre = _prefill(x, W, per_head=True)
    assert_parity(metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref), ("per-head", W))
    out32, _ = _prefill(x, W, per_head=True, out_dtype=torch.float32)
    assert_parity(metrics(out32.cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref), ("fp32 out", W))
    fused = to_dev(np.concatenate([x["q1"], x["q2"], x["k1"], x["k2"], x["v"]], axis=3))
    q1, q2, k1, k2, v = (fused[..., 0:64], fused[..., 64:128], fused[..., 128:192], fused[..., 192:256],
                         fused[..., 256:384])
    out_s = da.diffattn_fwd_prefill_ex(q1, q2, k1, k2, v, f32_dev(x["lam"]), f32_dev(x["gain"]), eps=x["eps"],
                                       scale=x["scale"], window=W)
    torch.cuda.synchronize()
    # Same kernel, same arithmetic: the layout and the missing o_pre change nothing.
    assert torch.equal(out_s, out)


def _window_rows(B, T, H, W, rng, n_random=40):
    rows = set()
    for b in {0, B - 1}:
        for h in {0, H - 1}:
            for i in (0, 1, W - 2, W - 1, W, W + 1, 127, 128, T // 2, T - W, T - 33, T - 1):
                if 0 <= i < T:
                    rows.add((b, i, h))
    for _ in range(n_random):
        rows.add((int(rng.integers(B)), int(rng.integers(T)), int(rng.integers(H))))
    return sorted(rows)


@pytest.mark.parametrize("B,T,H,W", [(1, 4096, 16, 128), (1, 8192, 16, 128), (2, 8192, 16, 1000),
                                     (1, 16384, 16, 4096)])
def test_prefill_window_large_sampled(B, T, H, W):
    _say("prefill window sampled rows", B, T, H, W)
    x = _inputs(B, T, H, seed=7 + W)
    out, o_pre = _prefill(x, W)
    assert bool(torch.isfinite(out.float()).all())
    rows = _window_rows(B, T, H, W, np.random.default_rng(T + W))
    o_ref, y_ref = _oracle_prefill(x, W, rows=rows)
    idx = torch.tensor(rows, dtype=torch.long, device="cuda")
    y = out[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy()
    o = o_pre[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy()
    m = metrics(y, y_ref, o, o_ref)
    _say("metrics", m)
    assert_parity(m, (B, T, H, W))


def test_prefill_window_properties():
    _say("prefill window: >= T equals causal, window 0 equals plain, old keys ignored")
    x = _inputs(1, 300, 2, seed=12)
    plain, pre_plain = _prefill(x, 0, ex=False)
    for W in (0, 300, 301, 5000):
        out, pre = _prefill(x, W)
        assert torch.equal(out, plain) and torch.equal(pre, pre_plain), W
    # keys and values older than every window are never read into a result
    W, cut = 40, 100
    out_a, pre_a = _prefill(x, W)
    xc = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
    for n in ("k1", "k2", "v"):
        xc[n][:, :cut] = synth.normal_bf16(998, 2, xc[n][:, :cut].shape)
    out_c, pre_c = _prefill(xc, W)
    first = cut + W - 1  # rows >= first see only positions >= cut
    assert torch.equal(out_a[:, first:], out_c[:, first:]) and torch.equal(pre_a[:, first:], pre_c[:, first:])
    assert not torch.equal(pre_a[:, :first], pre_c[:, :first])
    # window 1: every row is (1 - lambda) v_i
    x1 = _inputs(1, 150, 2, seed=13, lam_range=(0.2, 0.9))
    _, pre1 = _prefill(x1, 1, per_head=True)
    v = torch.from_numpy(synth.bf16_bits_to_f32(x1["v"])).cuda()
    lam = torch.from_numpy(x1["lam"].astype(np.float32)).cuda()
    assert float((pre1 - (1 - lam)[None, None, :, None] * v).abs().max()) < 1e-2


# ----------------------------- decode ------------------------------------

def _dec_inputs(B, L, H, seed, lam=0.8, lam_range=None):
    wl = Workload("dcase", "decode", B=B, T=L, H=H, seed=seed, lam=lam, lam_range=lam_range)
    return synth.make_decode_inputs(wl)


def _decode(x, seqlens=None, splits=0, window=0, ring=False, per_head=False, cache=None):
    q1, q2 = to_dev(x["q1"]), to_dev(x["q2"])
    src = cache if cache is not None else x
    k1, k2, v = (to_dev(src[n]) for n in ("k1", "k2", "v"))
    gain = f32_dev(x["gain"])
    lam = f32_dev(x["lam"]) if per_head else float(x["lam"][0])
    B, H, _ = x["q1"].shape
    sl = None if seqlens is None else torch.from_numpy(np.asarray(seqlens, np.int32)).cuda()
    o_pre = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    out = da.diffattn_fwd_decode_ex(q1, q2, k1, k2, v, lam, gain, eps=x["eps"], scale=x["scale"], seqlens=sl,
                                    num_splits=splits, o_pre=o_pre, window=window, kv_ring=ring)
    torch.cuda.synchronize()
    return out, o_pre


def _oracle_decode(x, seqlens, window, ring=False, cache=None):
    src = cache if cache is not None else x
    return oracle.decode(x["q1"], x["q2"], src["k1"], src["k2"], src["v"], x["lam"], x["gain"], x["eps"],
                         x["scale"], seqlens=seqlens, window=window, ring=ring)


@pytest.mark.parametrize("W", [1, 7, 128, 500, 4096])
def test_decode_window(W):
    _say("decode window", W)
    B, L, H = 6, 1500, 2
    x = _dec_inputs(B, L, H, seed=40 + W, lam_range=(0.2, 0.9))
    seqlens = [1500, 1, 0, 130, 700, 99999]
    o_ref, y_ref = _oracle_decode(x, seqlens, W)
    for s in (1, 3, 8, 16):
        out, o_pre = _decode(x, seqlens, splits=s, window=W, per_head=True)
        m = metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref)
        _say("splits", s, "metrics", m)
        assert_parity(m, ("decode window", W, "splits", s))
        assert bool((o_pre[2] == 0).all()) and bool((out[2] == 0).all())


def _ring_from_linear(t, n, L):
    r = np.zeros((t.shape[0], L) + t.shape[2:], t.dtype)
    for b in range(t.shape[0]):
        for p in range(max(0, int(n[b]) - L), int(n[b])):
            r[b, p % L] = t[b, p]
    return r


@pytest.mark.parametrize("L,W", [(128, 0), (128, 128), (128, 100), (1000, 1), (1000, 513)])
def test_decode_ring(L, W):
    _say("decode ring", L, W)
    N = 5000
    x = _dec_inputs(5, N, 2, seed=60 + L + W)
    n = np.array([0, L - 3, L, 3 * L + 17, N], np.int32)
    ring = {k: _ring_from_linear(x[k], n, L) for k in ("k1", "k2", "v")}
    o_ref, y_ref = _oracle_decode(x, n, W, ring=True, cache=ring)
    for s in (1, 8):
        out, o_pre = _decode(x, n, splits=s, window=W, ring=True, cache=ring)
        m = metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref)
        _say("splits", s, "metrics", m)
        assert_parity(m, ("ring", L, W, s))
        # the same positions read from a linear cache give the same bits
        out_l, pre_l = _decode(x, n, splits=s, window=W if W else L)
        assert torch.equal(out_l, out) and torch.equal(pre_l, o_pre)


def test_decode_window_equals_last_prefill_row():
    _say("decode window vs last prefill row")
    x = _inputs(2, 700, 2, seed=14)
    for W in (1, 64, 300):
        _, pre_p = _prefill(x, W)
        xd = dict(x, q1=np.ascontiguousarray(x["q1"][:, -1]), q2=np.ascontiguousarray(x["q2"][:, -1]))
        _, pre_d = _decode(xd, window=W)
        assert float((pre_d - pre_p[:, -1]).abs().max()) < 2e-3, W


def test_swa_workloads():
    """The sliding-window workloads the benchmark times, in its launch shapes."""
    wl = synth.WORKLOADS["swa_b1_t16384_h16_w128"]
    _say("workload", wl.name)
    x = synth.make_prefill_inputs(wl)
    out, o_pre = _prefill(x, wl.window)
    assert bool(torch.isfinite(out.float()).all())
    rows = _window_rows(wl.B, wl.T, wl.H, wl.window, np.random.default_rng(wl.seed), n_random=200)
    o_ref, y_ref = _oracle_prefill(x, wl.window, rows=rows)
    idx = torch.tensor(rows, dtype=torch.long, device="cuda")
    m = metrics(out[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy(), y_ref,
                o_pre[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy(), o_ref)
    _say("metrics", m)
    assert_parity(m, wl.name)

    wd = synth.WORKLOADS["swa_decode_b64_l4096_h16_w128"]
    _say("workload", wd.name)
    xd = synth.make_decode_inputs(wd)
    o_ref, y_ref = _oracle_decode(xd, None, wd.window)
    out, o_pre = _decode(xd, splits=wd.num_splits, window=wd.window)
    m = metrics(out.float().cpu().numpy(), y_ref, o_pre.cpu().numpy(), o_ref)
    _say("metrics", m)
    assert_parity(m, wd.name)
