"""Calls on a side stream: the binding's temporary buffers (the RoPE key
workspace, the decode split partials, outputs it allocates) belong to the
stream the kernels run on, so memory the caller allocates on another stream
right after the call never aliases a buffer those kernels still use."""
import numpy as np
import pytest

import synth
from tests.parity_util import f32_dev, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import differential_attention_causal_amd as da  # noqa: E402


def _say(*a):
    print("[case]", *a, flush=True)


def test_side_stream_prefill_rope_workspace():
    _say("side stream: RoPE prefill workspace, then a scribbled allocation on the current stream")
    wl = synth.WORKLOADS["prefill_b1_t4096_h16"]
    x = synth.make_prefill_inputs(wl)
    q1, q2, k1, k2, v = (to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v"))
    gain = f32_dev(x["gain"])
    kw = dict(eps=wl.eps, scale=wl.scale, rope=da.ROPE_HALF, rope_theta=5e5)
    ref = da.diffattn_fwd_prefill_ex(q1, q2, k1, k2, v, wl.lam, gain, **kw)
    torch.cuda.synchronize()
    need = da.diffattn_prefill_workspace_bytes(wl.B, wl.T, wl.H, rope=da.ROPE_HALF)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        out = da.diffattn_fwd_prefill_ex(q1, q2, k1, k2, v, wl.lam, gain, stream=side, **kw)
        junk = torch.empty(need, dtype=torch.uint8, device="cuda")
        junk.fill_(0x7F)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        del junk


def test_side_stream_decode_workspace():
    _say("side stream: decode partials, then a scribbled allocation on the current stream")
    wl = synth.WORKLOADS["decode_b64_l4096_h16"]
    x = synth.make_decode_inputs(wl)
    q1, q2, k1, k2, v = (to_dev(x[n]) for n in ("q1", "q2", "k1", "k2", "v"))
    gain = f32_dev(x["gain"])
    kw = dict(eps=wl.eps, scale=wl.scale, num_splits=wl.num_splits)
    ref = da.diffattn_fwd_decode(q1, q2, k1, k2, v, wl.lam, gain, **kw)
    torch.cuda.synchronize()
    need = da.diffattn_decode_workspace_bytes(wl.B, wl.H, wl.d_v, wl.num_splits)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        out = da.diffattn_fwd_decode(q1, q2, k1, k2, v, wl.lam, gain, stream=side, **kw)
        junk = torch.empty(need, dtype=torch.uint8, device="cuda")
        junk.fill_(0x7F)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        del junk
    assert np.isfinite(ref.float().cpu().numpy()).all()
