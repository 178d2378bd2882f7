"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, and rejects every invalid argument with its status code before any
HIP call (so nothing here needs a GPU: the fake pointers are never touched)."""
import ctypes
import os
import re

import pytest

import differential_attention_causal_amd as da

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "diffattn.h")

OK, ENULL, ESHAPE, EUNSUP, ELAYOUT, EWS, EHIP, EVALUE = range(8)
A = 0x10000  # 16-byte aligned fake device address, never dereferenced


def _declared():
    txt = open(HEADER).read()
    return re.findall(r"DIFFATTN_API\s+[\w\s\*]+?\b(diffattn_\w+)\s*\(", txt)


def test_header_symbols_exported():
    names = _declared()
    assert set(names) == {"diffattn_fwd_prefill", "diffattn_fwd_decode", "diffattn_decode_workspace_bytes",
                          "diffattn_fwd_prefill_ex", "diffattn_fwd_decode_ex", "diffattn_rope_apply",
                          "diffattn_fwd_decode_noalloc",
                          "diffattn_fwd_prefill_train", "diffattn_bwd_workspace_bytes", "diffattn_bwd_prefill",
                          "diffattn_fwd_prefill_train_ex", "diffattn_bwd_prefill_ex",
                          "diffattn_grouped_decode_workspace_bytes", "diffattn_fwd_grouped_decode",
                          "diffattn_grouped_workspace_bytes", "diffattn_fwd_grouped",
                          "diffattn_prefill_workspace_bytes", "diffattn_fwd_prefill_ws", "diffattn_prefill_prepare",
                          "diffattn_status_string", "diffattn_abi_version"}
    lib = ctypes.CDLL(da.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert da.diffattn_abi_version() == 112


def test_status_strings():
    for rc in range(8):
        s = da.diffattn_status_string(rc)
        assert s and (rc == 0) == (s == "ok")
    assert "unknown" in da.diffattn_status_string(99)


def _opt_call(fn, fn_ex, opt, args):
    if opt is None:
        return fn(*args)
    if opt == "null":
        return fn_ex(None, *args)
    o = da._Options(**{k: v for k, v in opt.items() if k != "reserved"})
    for i, r in enumerate(opt.get("reserved", ())):
        o.reserved[i] = r
    return fn_ex(ctypes.byref(o), *args)


def _prefill(opt=None, **kw):
    args = dict(q1=A, q2=A, k1=A, k2=A, v=A, st=None, B=1, T=128, H=2, dqk=64, dv=128, lam=0.5, lamh=None,
                gain=A, eps=1e-5, scale=0.0, out=A, odt=0, opre=None, stream=None)
    args.update(kw)
    return _opt_call(da._lib.diffattn_fwd_prefill, da._lib.diffattn_fwd_prefill_ex, opt, list(args.values()))


def _decode(opt=None, **kw):
    need = da.diffattn_decode_workspace_bytes(4, 2, 128, 8)
    args = dict(q1=A, q2=A, k1=A, k2=A, v=A, st=None, sl=None, B=4, L=100, H=2, dqk=64, dv=128, lam=0.8,
                lamh=None, gain=A, eps=1e-5, scale=0.0, splits=8, ws=A, wsb=need, out=A, odt=0, opre=None,
                stream=None)
    args.update(kw)
    return _opt_call(da._lib.diffattn_fwd_decode, da._lib.diffattn_fwd_decode_ex, opt, list(args.values()))


@pytest.mark.parametrize("kw,rc", [
    (dict(q1=None), ENULL), (dict(v=None), ENULL), (dict(gain=None), ENULL), (dict(out=None), ENULL),
    (dict(B=0), ESHAPE), (dict(T=0), ESHAPE), (dict(H=-1), ESHAPE), (dict(T=(1 << 22) + 1), ESHAPE),
    (dict(B=1 << 13, H=1 << 12), ESHAPE), (dict(B=4096, H=16, T=1 << 20), ESHAPE),
    (dict(dqk=128), EUNSUP), (dict(dv=64), EUNSUP),
    (dict(k2=A + 2), ELAYOUT), (dict(out=A + 8), ELAYOUT), (dict(opre=A + 4), ELAYOUT),
    (dict(lam=float("nan")), EVALUE), (dict(lam=float("inf")), EVALUE), (dict(eps=-1.0), EVALUE),
    (dict(eps=float("nan")), EVALUE), (dict(scale=float("nan")), EVALUE), (dict(odt=2), EVALUE),
])
def test_prefill_rejects(kw, rc):
    assert _prefill(**kw) == rc


def test_prefill_rejects_bad_strides():
    st = (da._Strides * 5)(*[da._Strides(128 * 2 * 64, 2 * 64, 64) for _ in range(5)])
    st[4] = da._Strides(128 * 2 * 128, 2 * 128, 124)  # not a multiple of 8
    assert _prefill(st=st) == ELAYOUT
    st[4] = da._Strides(-8, 256, 128)
    assert _prefill(st=st) == ELAYOUT


@pytest.mark.parametrize("kw,rc", [
    (dict(q2=None), ENULL), (dict(L=0), ESHAPE), (dict(L=(1 << 26) + 1), ESHAPE), (dict(dqk=32), EUNSUP),
    (dict(splits=65), EVALUE), (dict(ws=None), EWS), (dict(ws=A + 4), EWS), (dict(wsb=16), EWS),
    (dict(k1=A + 6), ELAYOUT), (dict(lam=float("nan")), EVALUE), (dict(odt=-1), EVALUE),
])
def test_decode_rejects(kw, rc):
    assert _decode(**kw) == rc


def test_workspace_bytes():
    assert da.diffattn_decode_workspace_bytes(64, 16, 128, 8) == 64 * 16 * 8 * 2 * 130 * 4
    assert da.diffattn_decode_workspace_bytes(64, 16, 128, 0) == da.diffattn_decode_workspace_bytes(64, 16, 128, 8)
    assert da.diffattn_decode_workspace_bytes(0, 16, 128, 8) == 0
    assert da.diffattn_decode_workspace_bytes(1, 1, 64, 8) == 0
    assert da.diffattn_decode_workspace_bytes(1, 1, 128, 65) == 0


# Options of the *_ex entry points.  Cases expected to pass validation are
# given an invalid shape instead, so every call stops before any HIP call.
@pytest.mark.parametrize("opt,rc", [
    (dict(window=-1), EVALUE), (dict(rope=3), EVALUE), (dict(rope=-1), EVALUE),
    (dict(kv_ring=1), EVALUE), (dict(reserved=(0, 1)), EVALUE), (dict(ws_prepared=1), EVALUE),
    (dict(rope=1), EVALUE), (dict(rope=2, rope_theta=-1.0), EVALUE), (dict(rope=1, rope_theta=float("inf")), EVALUE),
    (dict(rope=1, rope_theta=float("nan")), EVALUE), (dict(rope=1, rope_theta=1e4, rope_pos0=-1), EVALUE),
    (dict(window=5), ESHAPE), (dict(window=1 << 30), ESHAPE), ("null", ESHAPE), (dict(), ESHAPE),
    (dict(rope=1, rope_theta=5e5), ESHAPE), (dict(rope=2, rope_theta=1e4, rope_pos0=77, window=9), ESHAPE),
])
def test_prefill_ex_options(opt, rc):
    assert (_prefill(opt=opt, T=0) if rc == ESHAPE else _prefill(opt=opt)) == rc


@pytest.mark.parametrize("opt,rc", [
    (dict(window=-7), EVALUE), (dict(rope=9), EVALUE), (dict(reserved=(2, 0)), EVALUE), (dict(ws_prepared=1), EVALUE),
    (dict(kv_ring=1, window=101), EVALUE),
    (dict(rope=1, rope_theta=0.0), EVALUE),
    (dict(window=3), ESHAPE), (dict(kv_ring=1), ESHAPE), (dict(kv_ring=1, window=100), ESHAPE), ("null", ESHAPE),
    (dict(rope=1, rope_theta=5e5, kv_ring=1), ESHAPE),
])
def test_decode_ex_options(opt, rc):
    assert (_decode(opt=opt, L=0) if rc == ESHAPE else _decode(opt=opt)) == rc


def _prefill_ws(opt, ws=A, wsb=1 << 30, **kw):
    args = dict(q1=A, q2=A, k1=A, k2=A, v=A, st=None, B=1, T=128, H=2, dqk=64, dv=128, lam=0.5, lamh=None,
                gain=A, eps=1e-5, scale=0.0, out=A, odt=0, opre=None)
    args.update(kw)
    o = da._Options(**opt)
    return da._lib.diffattn_fwd_prefill_ws(ctypes.byref(o), *args.values(), ws, wsb, None)


def _vt_bytes(B, T, H):
    return B * H * (-(-T // 32)) * 8192  # fp16 V^T tiles of 32 keys x 128 channels


def test_prefill_workspace_bytes():
    one = -(-1 * 4096 * 16 * 64 * 2 // 256) * 256
    assert da.diffattn_prefill_workspace_bytes(1, 4096, 16, rope=1) == 2 * one + _vt_bytes(1, 4096, 16)
    assert da.diffattn_prefill_workspace_bytes(2, 77, 3, rope=2) == (2 * (-(-2 * 77 * 3 * 128 // 256) * 256)
                                                                    + _vt_bytes(2, 77, 3))
    assert da.diffattn_prefill_workspace_bytes(1, 4096, 16) == _vt_bytes(1, 4096, 16)  # no rope: V^T tiles only
    assert da.diffattn_prefill_workspace_bytes(0, 4096, 16, rope=1) == 0
    assert da.diffattn_prefill_workspace_bytes(1, (1 << 22) + 1, 16, rope=1) == 0
    assert da._lib.diffattn_prefill_workspace_bytes(None, 1, 128, 2) == _vt_bytes(1, 128, 2)  # NULL options: plain


@pytest.mark.parametrize("opt,kw,rc", [
    (dict(rope=1, rope_theta=5e5), dict(ws=None), EWS),         # rope needs the workspace
    (dict(rope=2, rope_theta=5e5), dict(ws=A + 16), EWS),       # 256-byte alignment
    (dict(rope=1, rope_theta=5e5), dict(wsb=2 * 128 * 2 * 64 * 2 - 1), EWS),
    (dict(rope=1, rope_theta=5e5), dict(T=0), ESHAPE),          # arguments checked before the workspace
    (dict(rope=1, rope_theta=-1.0), dict(), EVALUE),
    (dict(rope=1, rope_theta=5e5), dict(k1=A + 2), ELAYOUT),
    (dict(), dict(ws=None, T=0), ESHAPE),                        # no rope: the workspace is not needed
    (dict(ws_prepared=1), dict(ws=None), EWS),                   # a prepared workspace must be given
    (dict(ws_prepared=2), dict(), EVALUE),
    (dict(ws_prepared=1), dict(wsb=_vt_bytes(1, 128, 2) - 1), EWS),
])
def test_prefill_ws_rejects(opt, kw, rc):
    assert _prefill_ws(opt, **kw) == rc


def _prepare(opt=None, **kw):
    args = dict(k1=A, k2=A, v=A, st=None, B=1, T=128, H=2, dqk=64, dv=128, ws=A, wsb=1 << 30, stream=None)
    args.update(kw)
    o = None if opt is None else ctypes.byref(da._Options(**opt))
    return da._lib.diffattn_prefill_prepare(o, *args.values())


@pytest.mark.parametrize("opt,kw,rc", [
    (None, dict(k2=None), ENULL), (None, dict(v=None), ENULL), (None, dict(ws=None), EWS),
    (None, dict(T=0), ESHAPE), (None, dict(B=0), ESHAPE), (None, dict(dqk=32), EUNSUP),
    (None, dict(v=A + 8), ELAYOUT), (None, dict(ws=A + 16), EWS), (None, dict(wsb=_vt_bytes(1, 128, 2) - 1), EWS),
    (dict(rope=1, rope_theta=5e5), dict(wsb=_vt_bytes(1, 128, 2)), EWS),  # rotated keys need room too
    (dict(ws_prepared=1), dict(), EVALUE), (dict(kv_ring=1), dict(), EVALUE), (dict(rope=1), dict(), EVALUE),
    (dict(window=-2), dict(), EVALUE),
])
def test_prepare_rejects(opt, kw, rc):
    assert _prepare(opt, **kw) == rc


def test_options_layout():
    # The C struct: six 4-byte fields then int32 reserved[2], 32 bytes.
    assert ctypes.sizeof(da._Options) == 32
    assert [f[0] for f in da._Options._fields_] == ["window", "kv_ring", "rope", "rope_pos0", "rope_theta",
                                                    "ws_prepared", "reserved"]
    txt = open(HEADER).read()
    body = txt[txt.index("typedef struct {\n    int32_t window;"):txt.index("} diffattn_options;")]
    assert re.findall(r"(\w+)(?:\[\d\])?;", body) == ["window", "kv_ring", "rope", "rope_pos0", "rope_theta",
                                                       "ws_prepared", "reserved"]


def _rope_apply(**kw):
    args = dict(x=A, sx=None, out=A, so=None, B=2, T=5, H=3, d=64, mode=1, theta=5e5, pos0=0, ps=None, stream=None)
    args.update(kw)
    return da._lib.diffattn_rope_apply(*args.values())


@pytest.mark.parametrize("kw,rc", [
    (dict(x=None), ENULL), (dict(out=None), ENULL), (dict(B=0), ESHAPE), (dict(T=-1), ESHAPE),
    (dict(B=1 << 12, T=1 << 12, H=1 << 11), ESHAPE), (dict(d=128), EUNSUP), (dict(mode=0), EVALUE),
    (dict(mode=3), EVALUE), (dict(theta=0.0), EVALUE), (dict(theta=float("nan")), EVALUE), (dict(pos0=-5), EVALUE),
    (dict(x=A + 2), ELAYOUT), (dict(out=A + 8), ELAYOUT),
])
def test_rope_apply_rejects(kw, rc):
    assert _rope_apply(**kw) == rc


def test_rope_apply_rejects_bad_strides():
    assert _rope_apply(sx=ctypes.byref(da._Strides(960, 192, 60))) == ELAYOUT
    assert _rope_apply(so=ctypes.byref(da._Strides(960, -64, 64))) == ELAYOUT


def _train(**kw):
    args = dict(q1=A, q2=A, k1=A, k2=A, v=A, st=None, B=1, T=128, H=2, dqk=64, dv=128, lam=0.5, lamh=None,
                gain=A, eps=1e-5, scale=0.0, out=A, odt=0, opre=None, o1=A, o2=A, lse=A, stream=None)
    args.update(kw)
    return da._lib.diffattn_fwd_prefill_train(*args.values())


@pytest.mark.parametrize("kw,rc", [
    (dict(o1=None), ENULL), (dict(lse=None), ENULL), (dict(o2=A + 4), ELAYOUT), (dict(T=0), ESHAPE),
    (dict(dqk=32), EUNSUP), (dict(lam=float("nan")), EVALUE),
])
def test_train_forward_rejects(kw, rc):
    assert _train(**kw) == rc


def _bwd(**kw):
    need = da.diffattn_bwd_workspace_bytes(1, 128, 2, 128)
    args = dict(q1=A, q2=A, k1=A, k2=A, v=A, st=None, B=1, T=128, H=2, dqk=64, dv=128, lam=0.5, lamh=None,
                gain=A, eps=1e-5, scale=0.0, o1=A, o2=A, lse=A, dy=A, dyt=0, dq1=A, dq2=A, dk1=A, dk2=A, dvv=A,
                dlam=A, dgain=A, ws=A, wsb=need, stream=None)
    args.update(kw)
    return da._lib.diffattn_bwd_prefill(*args.values())


@pytest.mark.parametrize("kw,rc", [
    (dict(dy=None), ENULL), (dict(dlam=None), ENULL), (dict(o1=None), ENULL), (dict(B=0), ESHAPE),
    (dict(T=(1 << 22) + 1), ESHAPE), (dict(dv=64), EUNSUP), (dict(dk2=A + 4), ELAYOUT), (dict(dyt=3), EVALUE),
    (dict(eps=-1.0), EVALUE), (dict(ws=None), EWS), (dict(ws=A + 16), EWS), (dict(wsb=64), EWS),
])
def test_bwd_rejects(kw, rc):
    assert _bwd(**kw) == rc


# The variants of the training forward and backward: options checked like
# the forward's (invalid shapes elsewhere, so every call stops before HIP).
@pytest.mark.parametrize("opt,rc", [
    (dict(window=-1), EVALUE), (dict(rope=5), EVALUE), (dict(rope=1, rope_theta=0.0), EVALUE),
    (dict(kv_ring=1), EVALUE), (dict(ws_prepared=1), EVALUE), (dict(reserved=(0, 3)), EVALUE),
    (dict(window=64, rope=2, rope_theta=5e5, rope_pos0=9), ESHAPE), ("null", ESHAPE),
])
def test_train_and_bwd_ex_options(opt, rc):
    def call(fn, args):
        if opt == "null":
            return fn(None, *args)
        o = da._Options(**{k: v for k, v in opt.items() if k != "reserved"})
        for i, r in enumerate(opt.get("reserved", ())):
            o.reserved[i] = r
        return fn(ctypes.byref(o), *args)

    targs = dict(q1=A, q2=A, k1=A, k2=A, v=A, st=None, B=1, T=128, H=2, dqk=64, dv=128, lam=0.5, lamh=None,
                 gain=A, eps=1e-5, scale=0.0, out=A, odt=0, opre=None, o1=A, o2=A, lse=A, stream=None)
    bargs = dict(q1=A, q2=A, k1=A, k2=A, v=A, st=None, B=1, T=128, H=2, dqk=64, dv=128, lam=0.5, lamh=None,
                 gain=A, eps=1e-5, scale=0.0, o1=A, o2=A, lse=A, dy=A, dyt=0, dq1=A, dq2=A, dk1=A, dk2=A, dv_=A,
                 dlam=A, dgain=A, ws=A, wsb=1 << 30, stream=None)
    if rc == ESHAPE:
        targs["T"] = bargs["T"] = 0
    assert call(da._lib.diffattn_fwd_prefill_train_ex, list(targs.values())) == rc
    assert call(da._lib.diffattn_bwd_prefill_ex, list(bargs.values())) == rc


def test_bwd_workspace_bytes():
    n = da.diffattn_bwd_workspace_bytes(2, 100, 3, 128)
    rows = 2 * 100 * 3
    assert n >= rows * 128 * 2 + rows * 2 * 4 + 3 * ((200 + 63) // 64) * 129 * 4 and n % 256 == 0
    assert da.diffattn_bwd_workspace_bytes(0, 100, 3, 128) == 0
    assert da.diffattn_bwd_workspace_bytes(1, 100, 3, 64) == 0


def _grouped(**kw):
    need = da.diffattn_grouped_workspace_bytes(1, 128, 8, 3, 128)
    args = dict(q=A, k=A, v=A, st=None, B=1, T=128, nh=8, g=3, dqk=64, dv=128, lam=A, gate=None, scale=0.0, out=A,
                odt=0, ws=A, wsb=need, stream=None)
    args.update(kw)
    return da._lib.diffattn_fwd_grouped(*args.values())


@pytest.mark.parametrize("kw,rc", [
    (dict(q=None), ENULL), (dict(lam=None), ENULL), (dict(out=None), ENULL), (dict(B=0), ESHAPE),
    (dict(T=0), ESHAPE), (dict(nh=6), ESHAPE), (dict(g=0), ESHAPE), (dict(nh=9, g=2), OK - 99),
    (dict(dqk=128), EUNSUP), (dict(scale=float("nan")), EVALUE), (dict(odt=5), EVALUE), (dict(k=A + 2), ELAYOUT),
    (dict(gate=A + 4), ELAYOUT), (dict(ws=None), EWS), (dict(wsb=16), EWS),
])
def test_grouped_rejects(kw, rc):
    if rc == OK - 99:  # valid shape (9 heads, g = 2): stops at the workspace size instead
        assert _grouped(**kw) == EWS
    else:
        assert _grouped(**kw) == rc


def test_grouped_workspace_bytes():
    # fp32 head outputs, then 8 KiB fp16 V^T tiles per (b, head) and 32 keys
    assert da.diffattn_grouped_workspace_bytes(2, 100, 8, 3, 128) == 2 * 100 * 8 * 128 * 4 + 2 * 8 * 4 * 8192
    assert da.diffattn_grouped_workspace_bytes(2, 100, 8, 2, 128) == 0
    assert da.diffattn_grouped_workspace_bytes(2, 100, 8, 3, 64) == 0


def test_prefill_rejects_token_stride_at_limit():
    # a token stride of 2^25 elements would overflow the 32-bit per-lane
    # offsets of a 32-row tile; one step below is accepted by validation
    # (the call then stops at the invalid shape B=0 before any HIP call)
    big = 1 << 25
    st = (da._Strides * 5)(*[da._Strides(128 * big, big, 64) for _ in range(5)])
    assert _prefill(st=st) == ELAYOUT
    st = (da._Strides * 5)(*[da._Strides(128 * (big - 8), big - 8, 64) for _ in range(5)])
    assert _prefill(st=st, B=0) == ESHAPE


HARNESS = r"""
#include <stdio.h>
#include <stdlib.h>
#include "extent.h"
int main(int argc, char** argv) {
  for (int i = 1; i + 3 < argc; i += 4) {
    long long stride = atoll(argv[i]);
    int k0 = atoi(argv[i + 1]), kend = atoi(argv[i + 2]), row = atoi(argv[i + 3]);
    printf("%u\n", diffattn::rows_extent_bytes(stride, k0, kend, row));
  }
  return 0;
}
"""


def test_rows_extent_bytes_host(tmp_path):
    """The num_records of a buffer resource over rows k0 .. kend-1: exact below
    2^32 bytes, clamped above (a fused 12288-byte-row layout at 400K tokens
    spans 4.9 GB from the first row)."""
    import subprocess

    src = tmp_path / "h.cpp"
    src.write_text(HARNESS)
    exe = tmp_path / "h"
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-I",
                           os.path.join(ROOT, "differential_attention_causal_amd", "csrc"), str(src), "-o", str(exe)])
    cases = [(64, 0, 0, 64), (64, 5, 5, 64), (64, 0, 1, 64), (1024, 0, 128, 64), (6144, 0, 400000, 128),
             (6144, 399968, 400000, 128), (6144, 0, 349000, 64), (1 << 20, 0, 4096, 128), (8, 3, 10, 8)]
    out = subprocess.check_output([str(exe)] + [str(x) for c in cases for x in c], text=True).split()
    for (stride, k0, kend, row), got in zip(cases, out):
        exact = 0 if kend <= k0 else ((kend - k0 - 1) * stride + row) * 2
        assert int(got) == min(exact, 0xFFFFFFFF), (stride, k0, kend, row, got)


def _decode_noalloc(**kw):
    args = dict(opt=ctypes.byref(da._Options()), q1=A, q2=A, k1=A, k2=A, v=A, st=None, sl=None, B=4, L=100, H=2,
                dqk=64, dv=128, lam=0.8, lamh=None, gain=A, eps=1e-5, scale=0.0, splits=8, out=A, odt=0, opre=None,
                stream=None)
    args.update(kw)
    return da._lib.diffattn_fwd_decode_noalloc(*args.values())


@pytest.mark.parametrize("kw,rc", [
    (dict(q1=None), ENULL), (dict(out=None), ENULL), (dict(L=0), ESHAPE), (dict(dv=64), EUNSUP),
    (dict(splits=65), EVALUE), (dict(k1=A + 6), ELAYOUT), (dict(lam=float("nan")), EVALUE),
    # partials beyond the library's buffer: B*H*splits*2*130*4 > 16 MiB
    (dict(B=64, H=16, splits=64), EWS), (dict(B=4096, H=1, splits=8), EWS),
    # within the buffer, stopped by another invalid argument before any HIP call
    (dict(B=64, H=16, splits=8, odt=5), EVALUE),
])
def test_decode_noalloc_rejects(kw, rc):
    assert _decode_noalloc(**kw) == rc
    if rc == EWS:
        B, H, s = kw["B"], kw["H"], kw["splits"]
        assert da.diffattn_decode_workspace_bytes(B, H, 128, s) > da.DECODE_SCRATCH_BYTES


def _gdec(opt=None, **kw):
    need = da.diffattn_grouped_decode_workspace_bytes(2, 4, 128, 8)
    args = dict(q=A, k=A, v=A, st=None, sl=None, B=2, L=100, nh=4, g=1, dqk=64, dv=128, lam=A, gate=None, scale=0.0,
                splits=8, ws=A, wsb=need, out=A, odt=0, stream=None)
    args.update(kw)
    o = None if opt is None else ctypes.byref(da._Options(**opt))
    return da._lib.diffattn_fwd_grouped_decode(o, *args.values())


@pytest.mark.parametrize("opt,kw,rc", [
    (None, dict(q=None), ENULL), (None, dict(lam=None), ENULL), (None, dict(out=None), ENULL),
    (None, dict(B=0), ESHAPE), (None, dict(L=0), ESHAPE), (None, dict(nh=5), ESHAPE), (None, dict(g=0), ESHAPE),
    (None, dict(dqk=32), EUNSUP), (None, dict(dv=64), EUNSUP), (None, dict(splits=65), EVALUE),
    (None, dict(odt=2), EVALUE), (None, dict(scale=float("nan")), EVALUE), (None, dict(k=A + 2), ELAYOUT),
    (None, dict(gate=A + 4), ELAYOUT), (None, dict(sl=A + 2), ELAYOUT), (None, dict(ws=None), EWS),
    (None, dict(wsb=16), EWS), (dict(rope=1, rope_theta=5e5), dict(), EVALUE), (dict(ws_prepared=1), dict(), EVALUE),
    (dict(kv_ring=1, window=101), dict(), EVALUE), (dict(window=-3), dict(), EVALUE),
])
def test_grouped_decode_rejects(opt, kw, rc):
    assert _gdec(opt, **kw) == rc


def test_grouped_decode_workspace_bytes():
    assert da.diffattn_grouped_decode_workspace_bytes(64, 16, 128, 8) == 64 * 16 * 8 * 130 * 4
    assert da.diffattn_grouped_decode_workspace_bytes(64, 16, 128, 0) == 64 * 16 * 8 * 130 * 4
    assert da.diffattn_grouped_decode_workspace_bytes(0, 16, 128, 8) == 0
    assert da.diffattn_grouped_decode_workspace_bytes(1, 16, 64, 8) == 0
    assert da.diffattn_grouped_decode_workspace_bytes(1, 16, 128, 65) == 0
