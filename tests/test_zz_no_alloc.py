"""diffattn_fwd_decode_noalloc (no workspace, no allocation: the split partials
live in the library's per-device buffer) against diffattn_fwd_decode_ex with
a workspace, through the C ABI: two calls in a row, the second smaller, each
bitwise equal to the workspace decode on the same inputs and within the
acceptance bounds of the fp64 oracle; a size beyond the buffer is refused."""
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


def _dev(x, per_head):
    t = {n: to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v")}
    t["gain"] = f32_dev(x["gain"])
    t["lam"] = f32_dev(x["lam"]) if per_head else float(x["lam"][0])
    return t


def _call(fn, t, x, B, H, splits, seqlens, **kw):
    out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    o_pre = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    fn(t["q1"], t["q2"], t["k1"], t["k2"], t["v"], t["lam"], t["gain"], out=out, eps=x["eps"], scale=x["scale"],
       seqlens=seqlens, num_splits=splits, o_pre=o_pre, **kw)
    return out, o_pre


def test_noalloc_decode_two_calls():
    big = synth.WORKLOADS["decode_b64_l4096_h16"]
    xb = synth.make_decode_inputs(big)
    small = Workload("noalloc_small", "decode", B=3, T=777, H=2, seed=77, lam_range=(0.2, 0.9))
    xs = synth.make_decode_inputs(small)
    sl_small = [777, 5, 300]
    tb, ts = _dev(xb, False), _dev(xs, True)
    sl = torch.tensor(sl_small, dtype=torch.int32, device="cuda")
    _say("workspace decode, both sizes")
    ref_b = _call(da.diffattn_fwd_decode_ex, tb, xb, big.B, big.H, big.num_splits, None)
    ref_s = _call(da.diffattn_fwd_decode_ex, ts, xs, small.B, small.H, 4, sl, window=200)
    torch.cuda.synchronize()
    _say("no-allocation decode: B=64 L=4096 H=16 8 splits, then B=3 L=777 H=2 4 splits window 200")
    got_b = _call(da.diffattn_fwd_decode_noalloc, tb, xb, big.B, big.H, big.num_splits, None)
    got_s = _call(da.diffattn_fwd_decode_noalloc, ts, xs, small.B, small.H, 4, sl, window=200)
    torch.cuda.synchronize()
    for what, got, ref in (("big", got_b, ref_b), ("small", got_s, ref_s)):
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), what
    o_ref, y_ref = oracle.decode(xb["q1"], xb["q2"], xb["k1"], xb["k2"], xb["v"], xb["lam"], xb["gain"], xb["eps"],
                                 xb["scale"])
    m = metrics(got_b[0].cpu().numpy(), y_ref, got_b[1].cpu().numpy(), o_ref)
    _say("big vs oracle", m)
    assert_parity(m, "big")
    o_ref, y_ref = oracle.decode(xs["q1"], xs["q2"], xs["k1"], xs["k2"], xs["v"], xs["lam"], xs["gain"], xs["eps"],
                                 xs["scale"], seqlens=sl_small, window=200)
    m = metrics(got_s[0].cpu().numpy(), y_ref, got_s[1].cpu().numpy(), o_ref)
    _say("small vs oracle", m)
    assert_parity(m, "small")


def test_noalloc_decode_refuses_oversize():
    _say("no-allocation decode: partials beyond the buffer are refused")
    big = synth.WORKLOADS["decode_b64_l4096_h16"]
    xb = synth.make_decode_inputs(big)
    tb = _dev(xb, False)
    assert da.diffattn_decode_workspace_bytes(64, 16, 128, 64) > da.DECODE_SCRATCH_BYTES
    with pytest.raises(RuntimeError, match="workspace"):
        _call(da.diffattn_fwd_decode_noalloc, tb, xb, big.B, big.H, 64, None)
    got = _call(da.diffattn_fwd_decode_noalloc, tb, xb, big.B, big.H, 8, None)
    ref = _call(da.diffattn_fwd_decode_ex, tb, xb, big.B, big.H, 8, None)
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0])
    assert np.isfinite(got[0].cpu().numpy()).all()
