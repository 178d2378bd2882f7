"""Python binding of libdiffattn.so (causal differential attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/diffattn.h``; this module takes
torch tensors (device memory) and the current torch stream, checks dtypes and
shapes, passes raw pointers and strides through ctypes, and raises
``RuntimeError`` with the library's status text on any nonzero status.

There is no fallback: if the library is missing or fails to load, importing
this package raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

import torch  # first: the HIP runtime torch loads is the one the library binds to

__all__ = [
    "diffattn_fwd_prefill",
    "diffattn_fwd_prefill_ex",
    "diffattn_fwd_prefill_ws",
    "diffattn_prefill_workspace_bytes",
    "diffattn_fwd_decode",
    "diffattn_fwd_decode_ex",
    "diffattn_fwd_decode_noalloc",
    "diffattn_rope_apply",
    "diffattn_fwd_prefill_train",
    "diffattn_bwd_workspace_bytes",
    "diffattn_bwd_prefill",
    "diffattn_grouped_workspace_bytes",
    "diffattn_fwd_grouped",
    "diffattn_decode_workspace_bytes",
    "diffattn_status_string",
    "diffattn_abi_version",
    "LIB_PATH",
    "D_QK",
    "D_V",
]

D_QK = 64
D_V = 128
OUT_BF16 = 0
OUT_F32 = 1

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdiffattn.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libdiffattn.so is not built; run `python differential_attention_causal_amd/build.py` "
        "(or __graft_entry__.build()) first"
    )


ROPE_NONE = 0
ROPE_HALF = 1
ROPE_INTERLEAVED = 2


class _Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("t", ctypes.c_int64), ("h", ctypes.c_int64)]


class _Options(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("kv_ring", ctypes.c_int32), ("rope", ctypes.c_int32),
                ("rope_pos0", ctypes.c_int32), ("rope_theta", ctypes.c_float), ("ws_prepared", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 2)]


_lib = ctypes.CDLL(LIB_PATH)
_P, _I, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
_lib.diffattn_fwd_prefill.restype = _I
_lib.diffattn_fwd_prefill.argtypes = [_P, _P, _P, _P, _P, ctypes.POINTER(_Strides), _I, _I, _I, _I, _I,
                                      _F, _P, _P, _F, _F, _P, _I, _P, _P]
_lib.diffattn_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.diffattn_decode_workspace_bytes.argtypes = [_I, _I, _I, _I]
_lib.diffattn_fwd_decode.restype = _I
_lib.diffattn_fwd_decode.argtypes = [_P, _P, _P, _P, _P, ctypes.POINTER(_Strides), _P, _I, _I, _I, _I, _I,
                                     _F, _P, _P, _F, _F, _I, _P, ctypes.c_size_t, _P, _I, _P, _P]
_lib.diffattn_fwd_prefill_ex.restype = _I
_lib.diffattn_fwd_prefill_ex.argtypes = [ctypes.POINTER(_Options)] + _lib.diffattn_fwd_prefill.argtypes
_lib.diffattn_prefill_workspace_bytes.restype = ctypes.c_size_t
_lib.diffattn_prefill_workspace_bytes.argtypes = [ctypes.POINTER(_Options), _I, _I, _I]
_lib.diffattn_fwd_prefill_ws.restype = _I
_lib.diffattn_fwd_prefill_ws.argtypes = ([ctypes.POINTER(_Options)] + _lib.diffattn_fwd_prefill.argtypes[:-1]
                                         + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p])
_lib.diffattn_prefill_prepare.restype = _I
_lib.diffattn_prefill_prepare.argtypes = [ctypes.POINTER(_Options), _P, _P, _P, ctypes.POINTER(_Strides), _I, _I, _I,
                                          _I, _I, _P, ctypes.c_size_t, _P]
_lib.diffattn_fwd_decode_ex.restype = _I
_lib.diffattn_fwd_decode_ex.argtypes = [ctypes.POINTER(_Options)] + _lib.diffattn_fwd_decode.argtypes
_lib.diffattn_fwd_decode_noalloc.restype = _I
_lib.diffattn_fwd_decode_noalloc.argtypes = ([ctypes.POINTER(_Options)] + _lib.diffattn_fwd_decode.argtypes[:18]
                                             + _lib.diffattn_fwd_decode.argtypes[20:])
DECODE_SCRATCH_BYTES = 16 << 20
_lib.diffattn_rope_apply.restype = _I
_lib.diffattn_rope_apply.argtypes = [_P, ctypes.POINTER(_Strides), _P, ctypes.POINTER(_Strides), _I, _I, _I, _I,
                                     _I, ctypes.c_float, _I, _P, _P]
_lib.diffattn_fwd_prefill_train.restype = _I
_lib.diffattn_fwd_prefill_train.argtypes = _lib.diffattn_fwd_prefill.argtypes[:-1] + [_P, _P, _P, _P]
_lib.diffattn_fwd_prefill_train_ex.restype = _I
_lib.diffattn_fwd_prefill_train_ex.argtypes = [ctypes.POINTER(_Options)] + _lib.diffattn_fwd_prefill_train.argtypes
_lib.diffattn_bwd_workspace_bytes.restype = ctypes.c_size_t
_lib.diffattn_bwd_workspace_bytes.argtypes = [_I, _I, _I, _I]
_lib.diffattn_bwd_prefill.restype = _I
_lib.diffattn_bwd_prefill.argtypes = ([_P, _P, _P, _P, _P, ctypes.POINTER(_Strides), _I, _I, _I, _I, _I, ctypes.c_float,
                                      _P, _P, ctypes.c_float, ctypes.c_float, _P, _P, _P, _P, _I]
                                     + [_P] * 7 + [_P, ctypes.c_size_t, _P])
_lib.diffattn_bwd_prefill_ex.restype = _I
_lib.diffattn_bwd_prefill_ex.argtypes = [ctypes.POINTER(_Options)] + _lib.diffattn_bwd_prefill.argtypes
_lib.diffattn_grouped_workspace_bytes.restype = ctypes.c_size_t
_lib.diffattn_grouped_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
_lib.diffattn_fwd_grouped.restype = _I
_lib.diffattn_fwd_grouped.argtypes = [_P, _P, _P, ctypes.POINTER(_Strides), _I, _I, _I, _I, _I, _I, _P, _P,
                                      ctypes.c_float, _P, _I, _P, ctypes.c_size_t, _P]
_lib.diffattn_grouped_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.diffattn_grouped_decode_workspace_bytes.argtypes = [_I, _I, _I, _I]
_lib.diffattn_fwd_grouped_decode.restype = _I
_lib.diffattn_fwd_grouped_decode.argtypes = [ctypes.POINTER(_Options), _P, _P, _P, ctypes.POINTER(_Strides), _P, _I,
                                             _I, _I, _I, _I, _I, _P, _P, ctypes.c_float, _I, _P, ctypes.c_size_t,
                                             _P, _I, _P]
_lib.diffattn_status_string.restype = ctypes.c_char_p
_lib.diffattn_status_string.argtypes = [_I]
_lib.diffattn_abi_version.restype = _I
_lib.diffattn_abi_version.argtypes = []


def diffattn_status_string(status: int) -> str:
    return _lib.diffattn_status_string(int(status)).decode()


def diffattn_abi_version() -> int:
    return int(_lib.diffattn_abi_version())


def diffattn_decode_workspace_bytes(B: int, H: int, d_v: int = D_V, num_splits: int = 0) -> int:
    return int(_lib.diffattn_decode_workspace_bytes(B, H, d_v, num_splits))


def _check(rc: int) -> None:
    if rc != 0:
        raise RuntimeError(diffattn_status_string(rc))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides4(t: torch.Tensor) -> _Strides:
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, T, H, D] tensor with a contiguous last dimension")
    return _Strides(t.stride(0), t.stride(1), t.stride(2))


def _alloc_on(stream):
    """Context in which torch allocations belong to `stream` (when given): the
    caching allocator then reuses a temporary workspace, freed when the call
    returns, only for later work on that same stream, which the kernels
    enqueued on it precede."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _lambda_args(lam, H, device):
    """Scalar lambda -> (value, None); tensor [H] -> (0.0, fp32 device tensor)."""
    if isinstance(lam, torch.Tensor):
        if lam.shape != (H,) or lam.dtype != torch.float32 or lam.device != device or not lam.is_contiguous():
            raise ValueError("per-head lambda must be a contiguous fp32 [H] tensor on the inputs' device")
        return 0.0, lam
    return float(lam), None


def _out_code(dtype):
    if dtype == torch.bfloat16:
        return OUT_BF16
    if dtype == torch.float32:
        return OUT_F32
    raise ValueError("out dtype must be torch.bfloat16 or torch.float32")


def diffattn_fwd_prefill(q1, q2, k1, k2, v, lam, gain, eps=1e-5, scale=0.0, out=None,
                         out_dtype=torch.bfloat16, o_pre=None, stream=None):
    return _prefill(None, q1, q2, k1, k2, v, lam, gain, eps, scale, out, out_dtype, o_pre, stream)


def diffattn_fwd_prefill_ex(q1, q2, k1, k2, v, lam, gain, eps=1e-5, scale=0.0, out=None,
                            out_dtype=torch.bfloat16, o_pre=None, stream=None, window=0, rope=ROPE_NONE,
                            rope_theta=0.0, rope_pos0=0, workspace=True):
    """diffattn_fwd_prefill with variants: window > 0 is a sliding window
    (query i attends keys i-window+1 .. i); rope selects the rotary prologue.
    workspace: with rope on, True (default) runs diffattn_fwd_prefill_ws with a
    workspace from torch's allocator (keys rotated once), a uint8 device tensor
    runs it with that buffer, and False runs diffattn_fwd_prefill_ex (the keys
    rotated inside the kernels)."""
    opt = _Options(window=int(window), rope=int(rope), rope_pos0=int(rope_pos0), rope_theta=float(rope_theta))
    ws = None
    if int(rope) != ROPE_NONE and workspace is not False:
        B, T, H, _ = q1.shape
        need = diffattn_prefill_workspace_bytes(B, T, H, rope=rope)
        if isinstance(workspace, torch.Tensor):
            if workspace.dtype != torch.uint8 or not workspace.is_cuda or workspace.numel() < need:
                raise ValueError("workspace must be a uint8 device tensor of at least %d bytes" % need)
            ws = workspace
        else:
            with _alloc_on(stream):
                ws = torch.empty(need, dtype=torch.uint8, device=q1.device)
    return _prefill(opt, q1, q2, k1, k2, v, lam, gain, eps, scale, out, out_dtype, o_pre, stream, ws=ws)


def diffattn_fwd_prefill_ws(q1, q2, k1, k2, v, lam, gain, workspace, eps=1e-5, scale=0.0, out=None,
                            out_dtype=torch.bfloat16, o_pre=None, stream=None, window=0, rope=ROPE_NONE,
                            rope_theta=0.0, rope_pos0=0, prepared=False):
    """diffattn_fwd_prefill_ex with a caller's workspace (uint8 device tensor of
    diffattn_prefill_workspace_bytes(...) bytes; may be None without rope).
    prepared: the workspace already holds what diffattn_prefill_prepare wrote
    for these keys, values and options; only the prefill kernel runs."""
    opt = _Options(window=int(window), rope=int(rope), rope_pos0=int(rope_pos0), rope_theta=float(rope_theta),
                   ws_prepared=1 if prepared else 0)
    return _prefill(opt, q1, q2, k1, k2, v, lam, gain, eps, scale, out, out_dtype, o_pre, stream,
                    ws=workspace if workspace is not None else False)


def diffattn_prefill_prepare(k1, k2, v, workspace, stream=None, window=0, rope=ROPE_NONE, rope_theta=0.0,
                             rope_pos0=0):
    """The pre-pass of diffattn_fwd_prefill_ws alone (rotated keys with rope,
    fp16 V^T tiles) into `workspace`, for later calls with prepared=True on
    the same k1, k2, v and options."""
    B, T, H, d_qk = k1.shape
    d_v = v.shape[3]
    for t in (k1, k2, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise ValueError("k1, k2, v must be bf16 device tensors")
    if tuple(k2.shape) != (B, T, H, d_qk) or tuple(v.shape[:3]) != (B, T, H):
        raise ValueError("k1, k2 must share one shape and v be [B, T, H, d_v]")
    if workspace is None or workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise ValueError("workspace must be a uint8 device tensor")
    opt = _Options(window=int(window), rope=int(rope), rope_pos0=int(rope_pos0), rope_theta=float(rope_theta))
    st = (_Strides * 5)(*([_strides4(k1)] * 2 + [_strides4(t) for t in (k1, k2, v)]))
    rc = _lib.diffattn_prefill_prepare(ctypes.byref(opt), _ptr(k1), _ptr(k2), _ptr(v), st, B, T, H, d_qk, d_v,
                                       _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc)
    return workspace


def diffattn_prefill_workspace_bytes(B, T, H, rope=ROPE_NONE):
    """Workspace bytes diffattn_fwd_prefill_ws needs (0 without rope)."""
    opt = _Options(rope=int(rope), rope_theta=1.0)
    return int(_lib.diffattn_prefill_workspace_bytes(ctypes.byref(opt), int(B), int(T), int(H)))


def _prefill(opt, q1, q2, k1, k2, v, lam, gain, eps, scale, out, out_dtype, o_pre, stream, train=None, ws=None):
    """Causal differential-attention prefill.

    q1, q2, k1, k2: bf16 [B, T, H, 64]; v: bf16 [B, T, H, 128] (any strides with
    a contiguous last dimension).  lam: float, or fp32 [H] device tensor.
    gain: fp32 [H, 128].  out: optional preallocated [B, T, H, 128] output of
    ``out_dtype``; o_pre: optional fp32 [B, T, H, 128] for the pre-norm output.
    Returns out.  Runs asynchronously on ``stream`` (default: current stream).
    """
    B, T, H, d_qk = q1.shape
    d_v = v.shape[3]
    for t in (q1, q2, k1, k2, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise ValueError("q1, q2, k1, k2, v must be bf16 device tensors")
    for t in (q2, k1, k2):
        if tuple(t.shape) != (B, T, H, d_qk):
            raise ValueError("q1, q2, k1, k2 must share one shape")
    if tuple(v.shape[:3]) != (B, T, H):
        raise ValueError("v must be [B, T, H, d_v]")
    if gain.dtype != torch.float32 or tuple(gain.shape) != (H, d_v) or not gain.is_contiguous():
        raise ValueError("gain must be a contiguous fp32 [H, d_v] tensor")
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((B, T, H, d_v), dtype=out_dtype, device=q1.device)
    if tuple(out.shape) != (B, T, H, d_v) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, T, H, d_v] tensor")
    if o_pre is not None and (o_pre.dtype != torch.float32 or tuple(o_pre.shape) != (B, T, H, d_v)
                              or not o_pre.is_contiguous()):
        raise ValueError("o_pre must be a contiguous fp32 [B, T, H, d_v] tensor")
    lam_v, lam_t = _lambda_args(lam, H, q1.device)
    st = (_Strides * 5)(*[_strides4(t) for t in (q1, q2, k1, k2, v)])
    args = (_ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), _ptr(v), st, B, T, H, d_qk, d_v, lam_v, _ptr(lam_t),
            _ptr(gain), float(eps), float(scale), _ptr(out), _out_code(out.dtype), _ptr(o_pre), _stream(stream))
    if train is not None and opt is not None:
        rc = _lib.diffattn_fwd_prefill_train_ex(ctypes.byref(opt), *args[:-1], *(_ptr(t) for t in train), args[-1])
    elif train is not None:
        rc = _lib.diffattn_fwd_prefill_train(*args[:-1], *(_ptr(t) for t in train), args[-1])
    elif opt is None:
        rc = _lib.diffattn_fwd_prefill(*args)
    elif ws is not None:
        # ws False: the _ws entry point with no workspace (the library's checks apply)
        wsp, wsn = (None, 0) if ws is False else (_ptr(ws), ws.numel())
        rc = _lib.diffattn_fwd_prefill_ws(ctypes.byref(opt), *args[:-1], wsp, wsn, args[-1])
    else:
        rc = _lib.diffattn_fwd_prefill_ex(ctypes.byref(opt), *args)
    _check(rc)
    return out


def diffattn_fwd_decode(q1, q2, k1, k2, v, lam, gain, eps=1e-5, scale=0.0, seqlens=None, num_splits=0,
                        workspace=None, out=None, out_dtype=torch.bfloat16, o_pre=None, stream=None):
    return _decode(None, q1, q2, k1, k2, v, lam, gain, eps, scale, seqlens, num_splits, workspace, out,
                   out_dtype, o_pre, stream)


def diffattn_fwd_decode_ex(q1, q2, k1, k2, v, lam, gain, eps=1e-5, scale=0.0, seqlens=None, num_splits=0,
                           workspace=None, out=None, out_dtype=torch.bfloat16, o_pre=None, stream=None,
                           window=0, kv_ring=False, rope=ROPE_NONE, rope_theta=0.0, rope_pos0=0):
    """diffattn_fwd_decode with variants: window > 0 attends only the last
    `window` positions; kv_ring treats each sequence's L cache slots as a ring
    (position p in slot p % L, seqlens may exceed L)."""
    opt = _Options(window=int(window), kv_ring=int(bool(kv_ring)), rope=int(rope), rope_pos0=int(rope_pos0),
                   rope_theta=float(rope_theta))
    return _decode(opt, q1, q2, k1, k2, v, lam, gain, eps, scale, seqlens, num_splits, workspace, out,
                   out_dtype, o_pre, stream)


def diffattn_fwd_decode_noalloc(q1, q2, k1, k2, v, lam, gain, out, eps=1e-5, scale=0.0, seqlens=None,
                                num_splits=0, o_pre=None, stream=None, window=0, kv_ring=False, rope=ROPE_NONE,
                                rope_theta=0.0, rope_pos0=0):
    """diffattn_fwd_decode_ex with no workspace and no allocation (for callers
    that cannot allocate): the split partials live in the library's per-device
    buffer of DECODE_SCRATCH_BYTES; `out` (and `o_pre`) must be given.  Calls
    that overlap on one device race on that buffer."""
    if out is None:
        raise ValueError("out must be given: this entry point allocates nothing")
    opt = _Options(window=int(window), kv_ring=int(bool(kv_ring)), rope=int(rope), rope_pos0=int(rope_pos0),
                   rope_theta=float(rope_theta))
    return _decode(opt, q1, q2, k1, k2, v, lam, gain, eps, scale, seqlens, num_splits, None, out, out.dtype,
                   o_pre, stream, noalloc=True)


def _decode(opt, q1, q2, k1, k2, v, lam, gain, eps, scale, seqlens, num_splits, workspace, out, out_dtype,
            o_pre, stream, noalloc=False):
    """Single-query decode against a KV cache, split over cache positions.

    q1, q2: bf16 [B, H, 64] contiguous; k1, k2: bf16 cache [B, L, H, 64];
    v: bf16 cache [B, L, H, 128]; seqlens: optional int32 [B] device tensor.
    workspace: optional uint8 device tensor of at least
    ``diffattn_decode_workspace_bytes(B, H, 128, num_splits)`` bytes (allocated
    here through torch when omitted).  Returns out [B, H, 128].
    """
    B, H, d_qk = q1.shape
    L = k1.shape[1]
    d_v = v.shape[3]
    for t in (q1, q2, k1, k2, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise ValueError("q1, q2, k1, k2, v must be bf16 device tensors")
    if tuple(q2.shape) != (B, H, d_qk) or not q1.is_contiguous() or not q2.is_contiguous():
        raise ValueError("q1, q2 must be contiguous [B, H, d_qk]")
    if tuple(k1.shape) != (B, L, H, d_qk) or tuple(k2.shape) != (B, L, H, d_qk) or tuple(v.shape[:3]) != (B, L, H):
        raise ValueError("cache shapes disagree")
    if gain.dtype != torch.float32 or tuple(gain.shape) != (H, d_v) or not gain.is_contiguous():
        raise ValueError("gain must be a contiguous fp32 [H, d_v] tensor")
    if seqlens is not None and (seqlens.dtype != torch.int32 or tuple(seqlens.shape) != (B,)
                                or not seqlens.is_cuda):
        raise ValueError("seqlens must be an int32 [B] device tensor")
    need = diffattn_decode_workspace_bytes(B, H, d_v, num_splits)
    if workspace is None and not noalloc:
        with _alloc_on(stream):
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((B, H, d_v), dtype=out_dtype, device=q1.device)
    if tuple(out.shape) != (B, H, d_v) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, H, d_v] tensor")
    if o_pre is not None and (o_pre.dtype != torch.float32 or tuple(o_pre.shape) != (B, H, d_v)
                              or not o_pre.is_contiguous()):
        raise ValueError("o_pre must be a contiguous fp32 [B, H, d_v] tensor")
    lam_v, lam_t = _lambda_args(lam, H, q1.device)
    st = (_Strides * 3)(*[_strides4(t) for t in (k1, k2, v)])
    head = (_ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), _ptr(v), st, _ptr(seqlens), B, L, H, d_qk, d_v, lam_v,
            _ptr(lam_t), _ptr(gain), float(eps), float(scale), int(num_splits))
    tail = (_ptr(out), _out_code(out.dtype), _ptr(o_pre), _stream(stream))
    if noalloc:
        rc = _lib.diffattn_fwd_decode_noalloc(ctypes.byref(opt), *head, *tail)
        _check(rc)
        return out
    args = head + (_ptr(workspace), workspace.numel() * workspace.element_size()) + tail
    rc = _lib.diffattn_fwd_decode(*args) if opt is None else _lib.diffattn_fwd_decode_ex(ctypes.byref(opt), *args)
    _check(rc)
    return out


def diffattn_rope_apply(x, mode, theta, pos0=0, pos_start=None, out=None, stream=None):
    """Rotary embedding of a bf16 [B, T, H, 64] device tensor, the rotation the
    *_ex entry points apply with ``rope=mode``: token t of batch row b at
    position pos0 + pos_start[b] + t.  pos_start: optional int32 [B] device
    tensor.  out: optional destination (may be x, for in place); returns out."""
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 4:
        raise ValueError("x must be a bf16 [B, T, H, d] device tensor")
    B, T, H, d = x.shape
    if out is None:
        with _alloc_on(stream):
            out = torch.empty_like(x, memory_format=torch.contiguous_format)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (B, T, H, d):
        raise ValueError("out must be a bf16 tensor shaped like x")
    if pos_start is not None and (pos_start.dtype != torch.int32 or tuple(pos_start.shape) != (B,)
                                  or not pos_start.is_cuda):
        raise ValueError("pos_start must be an int32 [B] device tensor")
    sx, so = _strides4(x), _strides4(out)
    rc = _lib.diffattn_rope_apply(_ptr(x), ctypes.byref(sx), _ptr(out), ctypes.byref(so), B, T, H, d, int(mode),
                                  float(theta), int(pos0), _ptr(pos_start), _stream(stream))
    _check(rc)
    return out


def _variant_options(window, rope, rope_theta, rope_pos0):
    if int(window) == 0 and int(rope) == ROPE_NONE:
        return None
    return _Options(window=int(window), rope=int(rope), rope_pos0=int(rope_pos0), rope_theta=float(rope_theta))


def diffattn_fwd_prefill_train(q1, q2, k1, k2, v, lam, gain, eps=1e-5, scale=0.0, out=None,
                               out_dtype=torch.bfloat16, o_pre=None, stream=None, window=0, rope=ROPE_NONE,
                               rope_theta=0.0, rope_pos0=0):
    """Causal prefill that also returns what diffattn_bwd_prefill needs:
    (out, o1, o2, lse) with o1, o2 fp32 [B, T, H, 128] (each map's normalised
    output) and lse fp32 [B, T, H, 2] (base-2 log-sum-exp per map).  window,
    rope, rope_theta, rope_pos0: the variants (diffattn_fwd_prefill_train_ex);
    give the backward the same ones."""
    opt = _variant_options(window, rope, rope_theta, rope_pos0)
    B, T, H, _ = q1.shape
    with _alloc_on(stream):
        o1 = torch.empty((B, T, H, D_V), dtype=torch.float32, device=q1.device)
        o2 = torch.empty_like(o1)
        lse = torch.empty((B, T, H, 2), dtype=torch.float32, device=q1.device)
    out = _prefill(opt, q1, q2, k1, k2, v, lam, gain, eps, scale, out, out_dtype, o_pre, stream,
                   train=(o1, o2, lse))
    return out, o1, o2, lse


def diffattn_bwd_workspace_bytes(B: int, T: int, H: int, d_v: int = D_V) -> int:
    return int(_lib.diffattn_bwd_workspace_bytes(B, T, H, d_v))


def diffattn_bwd_prefill(q1, q2, k1, k2, v, lam, gain, o1, o2, lse, dy, eps=1e-5, scale=0.0, workspace=None,
                         grads=None, stream=None, window=0, rope=ROPE_NONE, rope_theta=0.0, rope_pos0=0):
    """Gradients of sum(y * dy) for the causal prefill.  dy: bf16 or fp32
    [B, T, H, 128], contiguous.  o1, o2, lse: diffattn_fwd_prefill_train's
    outputs (run with the same window and rope options).  Returns a dict of
    fp32 tensors dq1, dq2, dk1, dk2 ([B, T, H, 64], the gradients of the
    unrotated inputs), dv ([B, T, H, 128]), dlam ([H], per head) and dgain
    ([H, 128]); pass `grads` (such a dict) to write into preallocated
    tensors."""
    opt = _variant_options(window, rope, rope_theta, rope_pos0)
    B, T, H, d_qk = q1.shape
    d_v = v.shape[3]
    for t in (q1, q2, k1, k2, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise ValueError("q1, q2, k1, k2, v must be bf16 device tensors")
    if dy.dtype not in (torch.bfloat16, torch.float32) or tuple(dy.shape) != (B, T, H, d_v) or not dy.is_contiguous():
        raise ValueError("dy must be a contiguous bf16 or fp32 [B, T, H, d_v] tensor")
    for t, shp in ((o1, (B, T, H, d_v)), (o2, (B, T, H, d_v)), (lse, (B, T, H, 2))):
        if t.dtype != torch.float32 or tuple(t.shape) != shp or not t.is_contiguous():
            raise ValueError("o1, o2, lse must be diffattn_fwd_prefill_train's outputs")
    if gain.dtype != torch.float32 or tuple(gain.shape) != (H, d_v) or not gain.is_contiguous():
        raise ValueError("gain must be a contiguous fp32 [H, d_v] tensor")
    if grads is None:
        f = dict(dtype=torch.float32, device=q1.device)
        with _alloc_on(stream):
            grads = {"dq1": torch.empty((B, T, H, d_qk), **f), "dq2": torch.empty((B, T, H, d_qk), **f),
                     "dk1": torch.empty((B, T, H, d_qk), **f), "dk2": torch.empty((B, T, H, d_qk), **f),
                     "dv": torch.empty((B, T, H, d_v), **f), "dlam": torch.empty((H,), **f),
                     "dgain": torch.empty((H, d_v), **f)}
    need = diffattn_bwd_workspace_bytes(B, T, H, d_v)
    if workspace is None:
        with _alloc_on(stream):
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q1.device)
    lam_v, lam_t = _lambda_args(lam, H, q1.device)
    st = (_Strides * 5)(*[_strides4(t) for t in (q1, q2, k1, k2, v)])
    g = grads
    args = (_ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), _ptr(v), st, B, T, H, d_qk, d_v, lam_v, _ptr(lam_t), _ptr(gain),
            float(eps), float(scale), _ptr(o1), _ptr(o2), _ptr(lse), _ptr(dy), _out_code(dy.dtype), _ptr(g["dq1"]),
            _ptr(g["dq2"]), _ptr(g["dk1"]), _ptr(g["dk2"]), _ptr(g["dv"]), _ptr(g["dlam"]), _ptr(g["dgain"]),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if opt is None:
        rc = _lib.diffattn_bwd_prefill(*args)
    else:
        rc = _lib.diffattn_bwd_prefill_ex(ctypes.byref(opt), *args)
    _check(rc)
    return grads


def diffattn_grouped_workspace_bytes(B: int, T: int, n_heads: int, group: int, d_v: int = D_V) -> int:
    return int(_lib.diffattn_grouped_workspace_bytes(B, T, n_heads, group, d_v))


def diffattn_fwd_grouped(q, k, v, group, lambda_t, gate=None, scale=0.0, out=None, out_dtype=torch.bfloat16,
                         workspace=None, stream=None):
    """Grouped differential attention (signal heads first, signal head s paired
    with noise head n_S + s // group), token-wise lambda_t (fp32 [B, T, n_S]),
    optional bf16 gate logits [B, T, n_S, 128].  q, k: bf16 [B, T, n_heads, 64];
    v: bf16 [B, T, n_heads, 128].  Returns out [B, T, n_S, 128]."""
    B, T, n_heads, d_qk = q.shape
    d_v = v.shape[3]
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise ValueError("q, k, v must be bf16 device tensors")
    if group < 1 or n_heads % (group + 1):
        raise ValueError("n_heads must be a multiple of group + 1")
    n_S = group * (n_heads // (group + 1))
    if (lambda_t.dtype != torch.float32 or tuple(lambda_t.shape) != (B, T, n_S) or not lambda_t.is_contiguous()):
        raise ValueError("lambda_t must be a contiguous fp32 [B, T, n_S] tensor")
    if gate is not None and (gate.dtype != torch.bfloat16 or tuple(gate.shape) != (B, T, n_S, d_v)
                             or not gate.is_contiguous()):
        raise ValueError("gate must be a contiguous bf16 [B, T, n_S, d_v] tensor")
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((B, T, n_S, d_v), dtype=out_dtype, device=q.device)
    need = diffattn_grouped_workspace_bytes(B, T, n_heads, group, d_v)
    if workspace is None:
        with _alloc_on(stream):
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = (_Strides * 3)(*[_strides4(t) for t in (q, k, v)])
    rc = _lib.diffattn_fwd_grouped(_ptr(q), _ptr(k), _ptr(v), st, B, T, n_heads, int(group), d_qk, d_v,
                                   _ptr(lambda_t), _ptr(gate), float(scale), _ptr(out), _out_code(out.dtype),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc)
    return out


def diffattn_grouped_decode_workspace_bytes(B, n_heads, d_v=D_V, num_splits=0):
    return int(_lib.diffattn_grouped_decode_workspace_bytes(int(B), int(n_heads), int(d_v), int(num_splits)))


def diffattn_fwd_grouped_decode(q, k, v, group, lambda_t, gate=None, scale=0.0, seqlens=None, num_splits=0,
                                out=None, out_dtype=torch.bfloat16, workspace=None, stream=None, window=0,
                                kv_ring=False):
    """Single-query decode of grouped differential attention: q bf16
    [B, n_heads, 64] (each sequence's newest token), caches k bf16
    [B, L, n_heads, 64] and v bf16 [B, L, n_heads, 128], seqlens optional
    int32 [B] device tensor, lambda_t fp32 [B, n_S], optional gate bf16
    [B, n_S, 128] logits.  Returns out [B, n_S, 128]."""
    B, n_heads, d_qk = q.shape
    L = k.shape[1]
    d_v = v.shape[3]
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise ValueError("q, k, v must be bf16 device tensors")
    if not q.is_contiguous() or tuple(k.shape) != (B, L, n_heads, d_qk) or tuple(v.shape[:3]) != (B, L, n_heads):
        raise ValueError("q must be a contiguous [B, n_heads, d_qk] tensor and k, v [B, L, n_heads, d] caches")
    if group < 1 or n_heads % (group + 1):
        raise ValueError("n_heads must be a multiple of group + 1")
    n_S = group * (n_heads // (group + 1))
    if lambda_t.dtype != torch.float32 or tuple(lambda_t.shape) != (B, n_S) or not lambda_t.is_contiguous():
        raise ValueError("lambda_t must be a contiguous fp32 [B, n_S] tensor")
    if gate is not None and (gate.dtype != torch.bfloat16 or tuple(gate.shape) != (B, n_S, d_v)
                             or not gate.is_contiguous()):
        raise ValueError("gate must be a contiguous bf16 [B, n_S, d_v] tensor")
    if seqlens is not None and (seqlens.dtype != torch.int32 or tuple(seqlens.shape) != (B,) or not seqlens.is_cuda):
        raise ValueError("seqlens must be an int32 [B] device tensor")
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((B, n_S, d_v), dtype=out_dtype, device=q.device)
    need = diffattn_grouped_decode_workspace_bytes(B, n_heads, d_v, num_splits)
    if workspace is None:
        with _alloc_on(stream):
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    opt = _Options(window=int(window), kv_ring=int(bool(kv_ring)))
    st = (_Strides * 2)(*[_strides4(t) for t in (k, v)])
    rc = _lib.diffattn_fwd_grouped_decode(ctypes.byref(opt), _ptr(q), _ptr(k), _ptr(v), st, _ptr(seqlens), B, L,
                                          n_heads, int(group), d_qk, d_v, _ptr(lambda_t), _ptr(gate), float(scale),
                                          int(num_splits), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _ptr(out),
                                          _out_code(out.dtype), _stream(stream))
    _check(rc)
    return out


def default_scale(d_qk: int = D_QK) -> float:
    return 1.0 / math.sqrt(d_qk)
