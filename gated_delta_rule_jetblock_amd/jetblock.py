"""ctypes binding of libjetblock (include/jetblock.h).

Argument marshalling only: shapes and dtypes are read off torch tensors,
outputs and workspaces are allocated with torch on the tensors' device, and
every computation runs in the library's HIP kernels on the current torch
stream.  There is no fallback: if libjetblock.so is missing or fails to load,
importing this module raises, and a call on CPU tensors raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libjetblock.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "jetblock.h")

JB_OK, JB_ERR_INVALID_ARG, JB_ERR_UNSUPPORTED, JB_ERR_WORKSPACE, JB_ERR_HIP = range(5)
JB_BF16, JB_F32 = 0, 1
_DT = {torch.bfloat16: JB_BF16, torch.float32: JB_F32}
_TORCH = {JB_BF16: torch.bfloat16, JB_F32: torch.float32}


class JetBlockError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [{status}]")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "H", "dk", "dv", "d_model", "gen_hidden", "taps", "chunk",
                 "io_dtype", "out_dtype", "flags")]


def flag_segment(n: int) -> int:
    return (int(n) & 0xFFFF) << 8


if not os.path.exists(LIB_PATH):
    raise ImportError(f"libjetblock.so not built at {LIB_PATH}; run "
                      "`python -m gated_delta_rule_jetblock_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_S = ctypes.POINTER(Shape)
_SZ = ctypes.c_size_t
_lib.jb_status_string.argtypes = [ctypes.c_int]
_lib.jb_status_string.restype = ctypes.c_char_p
_lib.jb_last_error.argtypes = []
_lib.jb_last_error.restype = ctypes.c_char_p
_lib.jb_version.argtypes = []
_lib.jb_version.restype = ctypes.c_int32
_lib.jb_prefill_workspace_size.argtypes = [_S, ctypes.POINTER(_SZ)]
_lib.jb_decode_workspace_size.argtypes = [_S, ctypes.POINTER(_SZ)]
_lib.jb_prefill.argtypes = [_S] + [_P] * 15 + [_P, _SZ, _P]
_lib.jb_decode_step.argtypes = [_S] + [_P] * 15 + [_P, _SZ, _P]
_lib.jb_prefill_noalloc.argtypes = [_S] + [_P] * 15 + [_P]
_lib.jb_gen_taps.argtypes = [_S] + [_P] * 6 + [_P]
_lib.jb_gen_conv.argtypes = [_S] + [_P] * 9 + [_P]
_lib.jb_prologue.argtypes = [_S] + [_P] * 6 + [_P]
_lib.jb_probe_mfma.argtypes = [ctypes.c_int32, _P, _P, _P, _P]
_lib.jb_decode_update.argtypes = [_S] + [_P] * 11 + [_P]
_lib.jb_project_workspace_size.argtypes = [_S, ctypes.POINTER(_SZ)]
_lib.jb_prefill_from_x_workspace_size.argtypes = [_S, ctypes.POINTER(_SZ)]
_lib.jb_project.argtypes = [_S] + [_P] * 18 + [_P, _SZ, _P]
_lib.jb_prefill_from_x.argtypes = [_S] + [_P] * 17 + [_P, _SZ, _P]
_lib.jb_decode_step_from_x_workspace_size.argtypes = [_S, ctypes.POINTER(_SZ)]
_lib.jb_decode_step_from_x.argtypes = [_S] + [_P] * 17 + [_P, _SZ, _P]
_lib.jb_prefill_static_workspace_size.argtypes = [_S, ctypes.POINTER(_SZ)]
_lib.jb_prefill_static.argtypes = [_S] + [_P] * 17 + [_P, _SZ, _P]
_lib.jb_decode_step_static.argtypes = [_S] + [_P] * 17 + [_P]
_lib.jb_prefill_varlen_workspace_size.argtypes = [_S, ctypes.c_int64, ctypes.POINTER(_SZ)]
_lib.jb_prefill_varlen.argtypes = [_S, ctypes.c_int64] + [_P] * 16 + [_P, _SZ, _P]
_lib.jb_backward_workspace_size.argtypes = [_S, ctypes.POINTER(_SZ)]
_lib.jb_backward.argtypes = [_S] + [_P] * 27 + [_P, _SZ, _P]
for _f in ("jb_prefill_workspace_size", "jb_decode_workspace_size", "jb_prefill", "jb_prefill_noalloc",
           "jb_decode_step",
           "jb_gen_taps", "jb_gen_conv", "jb_prologue", "jb_probe_mfma", "jb_decode_update",
           "jb_project_workspace_size", "jb_prefill_from_x_workspace_size", "jb_project", "jb_prefill_from_x",
           "jb_decode_step_from_x_workspace_size", "jb_decode_step_from_x", "jb_prefill_static_workspace_size",
           "jb_prefill_static", "jb_decode_step_static", "jb_prefill_varlen_workspace_size",
           "jb_prefill_varlen", "jb_backward_workspace_size", "jb_backward"):
    getattr(_lib, _f).restype = ctypes.c_int


def declared_functions() -> list[str]:
    """Names of the functions include/jetblock.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jb_[a-z_0-9]+)\s*\(", text)) - {"jb_FLAG_SEGMENT"})


def library() -> ctypes.CDLL:
    return _lib


def version() -> int:
    return _lib.jb_version()


def last_error() -> str:
    return _lib.jb_last_error().decode()


def _check(status: int):
    if status != JB_OK:
        raise JetBlockError(status, f"{_lib.jb_status_string(status).decode()}: {last_error()}")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError("libjetblock takes device tensors; got a tensor on " + str(t.device))
    if not t.is_contiguous():
        raise ValueError("libjetblock takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def make_shape(B, T, H, dk, dv, d_model, io_dtype=JB_BF16, out_dtype=JB_F32, flags=0) -> Shape:
    return Shape(B, T, H, dk, dv, d_model, 32, 4, 64, io_dtype, out_dtype, flags)


def _io_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def prefill_workspace_size(shape: Shape) -> int:
    n = _SZ(0)
    _check(_lib.jb_prefill_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def decode_workspace_size(shape: Shape) -> int:
    n = _SZ(0)
    _check(_lib.jb_decode_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def workspace(nbytes: int, device) -> torch.Tensor:
    """A device byte buffer of at least nbytes (torch allocations are 256-byte aligned)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def prefill(x, q, k, v, alpha, beta, W1, W2, b1=None, b2=None, S0=None, conv_in=None, *,
            out_dtype=torch.float32, seg_len: int | None = None, o=None, S_final=None,
            conv_out=None, want_conv_out=True, ws=None, stream=None):
    """jb_prefill.  x [B,T,D], q,k [B,T,H,dk], v [B,T,H,dv], alpha,beta [B,T,H] f32.

    Returns dict(o, S_final, conv_out).  Outputs are allocated unless given.
    """
    B, T, D = x.shape
    H, dk = q.shape[2], q.shape[3]
    dv = v.shape[3]
    io = _io_code(x)
    shape = make_shape(B, T, H, dk, dv, D, io, _DT[out_dtype], flag_segment(seg_len) if seg_len else 0)
    dev = x.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    if S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if conv_out is None and want_conv_out:
        conv_out = torch.empty((B, 3, H, dv), dtype=x.dtype, device=dev)
    need = prefill_workspace_size(shape)
    if ws is None:
        ws = workspace(need, dev)
    _check(_lib.jb_prefill(ctypes.byref(shape), _ptr(x), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                           _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), _ptr(S0), _ptr(conv_in), _ptr(o),
                           _ptr(S_final), _ptr(conv_out), _ptr(ws), ws.numel(), _stream(stream)))
    return dict(o=o, S_final=S_final, conv_out=conv_out)


def prefill_noalloc(x, q, k, v, alpha, beta, W1, W2, b1=None, b2=None, S0=None, conv_in=None, *,
                    out_dtype=torch.float32, seg_len: int | None = None, o=None, S_final=None,
                    conv_out=None, want_conv_out=True, stream=None):
    """jb_prefill_noalloc: jb_prefill on the library's own per-device scratch array
    (NOALLOC_SCRATCH_BYTES).  Same arguments as prefill() without ws; outputs are
    allocated here unless given, so a caller that must not allocate passes o, S_final
    and conv_out (or want_conv_out=False)."""
    B, T, D = x.shape
    H, dk = q.shape[2], q.shape[3]
    dv = v.shape[3]
    shape = make_shape(B, T, H, dk, dv, D, _io_code(x), _DT[out_dtype], flag_segment(seg_len) if seg_len else 0)
    dev = x.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    if S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if conv_out is None and want_conv_out:
        conv_out = torch.empty((B, 3, H, dv), dtype=x.dtype, device=dev)
    _check(_lib.jb_prefill_noalloc(ctypes.byref(shape), _ptr(x), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                   _ptr(beta), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), _ptr(S0), _ptr(conv_in),
                                   _ptr(o), _ptr(S_final), _ptr(conv_out), _stream(stream)))
    return dict(o=o, S_final=S_final, conv_out=conv_out)


NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_step(S, cache, x_t, q_t, k_t, v_t, alpha_t, beta_t, W1, W2, b1=None, b2=None, *,
                out_dtype=torch.float32, S_out=None, cache_out=None, o=None, ws=None, stream=None):
    """jb_decode_step.  S [B,H,dk,dv] f32, cache [B,3,H,dv], x_t [B,D], q_t,k_t [B,H,dk],
    v_t [B,H,dv], alpha_t,beta_t [B,H].  In place on S and cache unless S_out/cache_out
    are given.  Returns dict(o, S, cache)."""
    B, D = x_t.shape
    H, dk = q_t.shape[1], q_t.shape[2]
    dv = v_t.shape[2]
    shape = make_shape(B, 1, H, dk, dv, D, _io_code(x_t), _DT[out_dtype])
    if S_out is None:
        S_out = S
    if cache_out is None:
        cache_out = cache
    if o is None:
        o = torch.empty((B, H, dv), dtype=out_dtype, device=x_t.device)
    if ws is None and decode_workspace_size(shape) > 0:
        ws = workspace(decode_workspace_size(shape), x_t.device)
    _check(_lib.jb_decode_step(ctypes.byref(shape), _ptr(S), _ptr(S_out), _ptr(cache), _ptr(cache_out),
                               _ptr(x_t), _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(alpha_t), _ptr(beta_t),
                               _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), _ptr(o), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream(stream)))
    return dict(o=o, S=S_out, cache=cache_out)


def decode_update(S, cache, q_t, k_t, v_t, alpha_t, beta_t, taps, *, d_model: int = 128,
                  out_dtype=torch.float32, S_out=None, cache_out=None, o=None, stream=None):
    """jb_decode_update: the state-update stage with taps [B,H,4] f32 precomputed.
    In place on S and cache unless S_out/cache_out are given."""
    B, H, dk = q_t.shape
    dv = v_t.shape[2]
    shape = make_shape(B, 1, H, dk, dv, d_model, _io_code(q_t), _DT[out_dtype])
    S_out = S if S_out is None else S_out
    cache_out = cache if cache_out is None else cache_out
    if o is None:
        o = torch.empty((B, H, dv), dtype=out_dtype, device=q_t.device)
    _check(_lib.jb_decode_update(ctypes.byref(shape), _ptr(S), _ptr(S_out), _ptr(cache), _ptr(cache_out),
                                 _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(alpha_t), _ptr(beta_t), _ptr(taps),
                                 _ptr(o), _stream(stream)))
    return dict(o=o, S=S_out, cache=cache_out)


def gen_taps(x, W1, W2, b1=None, b2=None, H: int | None = None, *, out=None, stream=None):
    """jb_gen_taps on x [B,T,D] -> taps [B,T,H,4] f32 (written into `out` when given)."""
    B, T, D = x.shape
    if H is None:
        H = W2.shape[0] // 4
    shape = make_shape(B, T, H, 32, 64, D, _io_code(x))
    taps = torch.empty((B, T, H, 4), dtype=torch.float32, device=x.device) if out is None else out
    _check(_lib.jb_gen_taps(ctypes.byref(shape), _ptr(x), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), _ptr(taps),
                            _stream(stream)))
    return taps


def gen_conv(x, W1, W2, v, b1=None, b2=None, conv_in=None, *, stream=None):
    """jb_gen_conv -> (taps [B,T,H,4], vconv [B,T,H,dv]) f32."""
    B, T, D = x.shape
    H, dv = v.shape[2], v.shape[3]
    shape = make_shape(B, T, H, 32, dv, D, _io_code(x))
    taps = torch.empty((B, T, H, 4), dtype=torch.float32, device=x.device)
    vconv = torch.empty((B, T, H, dv), dtype=torch.float32, device=x.device)
    _check(_lib.jb_gen_conv(ctypes.byref(shape), _ptr(x), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), _ptr(v),
                            _ptr(conv_in), _ptr(taps), _ptr(vconv), _stream(stream)))
    return taps, vconv


def prologue(q, k, alpha, *, stream=None):
    """jb_prologue -> (qhat, khat [B,T,H,dk] f32, g [B,T,H] f32)."""
    B, T, H, dk = q.shape
    shape = make_shape(B, T, H, dk, 64, 128, _io_code(q))
    qh = torch.empty((B, T, H, dk), dtype=torch.float32, device=q.device)
    kh = torch.empty_like(qh)
    g = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    _check(_lib.jb_prologue(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(alpha), _ptr(qh), _ptr(kh), _ptr(g),
                            _stream(stream)))
    return qh, kh, g


def probe_mfma(kind: int, A, B, *, stream=None):
    """jb_probe_mfma: D = A B for A [16,32], B [32,16] f32 device tensors."""
    D = torch.empty((16, 16), dtype=torch.float32, device=A.device)
    _check(_lib.jb_probe_mfma(int(kind), _ptr(A), _ptr(B), _ptr(D), _stream(stream)))
    return D


def project_workspace_size(shape: Shape) -> int:
    n = _SZ(0)
    _check(_lib.jb_project_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def prefill_from_x_workspace_size(shape: Shape) -> int:
    n = _SZ(0)
    _check(_lib.jb_prefill_from_x_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def _proj_shape(x, Wq, Wv, Wa, seg_len=None, out_dtype=torch.float32):
    B, T, D = x.shape
    H = Wa.shape[0]
    dk = Wq.shape[0] // H
    dv = Wv.shape[0] // H
    return make_shape(B, T, H, dk, dv, D, JB_BF16, _DT[out_dtype],
                      flags=flag_segment(seg_len) if seg_len else 0)


def project(x, Wq, Wk, Wv, Wa, Wb, W1, W2, ba=None, bb=None, b1=None, b2=None, *, ws=None, stream=None):
    """jb_project.  x [B,T,D] bf16; Wq, Wk [H*dk,D], Wv [H*dv,D], Wa, Wb [H,D], W1 [32,D], W2 [4H,32]
    bf16.  Returns dict(q, k [B,T,H,dk], v [B,T,H,dv] bf16, alpha, beta [B,T,H], taps [B,T,H,4] f32)."""
    shape = _proj_shape(x, Wq, Wv, Wa)
    B, T, H, dk, dv = shape.B, shape.T, shape.H, shape.dk, shape.dv
    dev = x.device
    q = torch.empty((B, T, H, dk), dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    v = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    alpha = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    beta = torch.empty_like(alpha)
    taps = torch.empty((B, T, H, 4), dtype=torch.float32, device=dev)
    # the projection kernel takes no workspace (jb_project_workspace_size is 0)
    _check(_lib.jb_project(ctypes.byref(shape), _ptr(x), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wa), _ptr(ba),
                           _ptr(Wb), _ptr(bb), _ptr(W1), _ptr(b1), _ptr(W2),
                           _ptr(b2), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(taps), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream(stream)))
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, taps=taps)


def prefill_from_x(x, Wq, Wk, Wv, Wa, Wb, W1, W2, ba=None, bb=None, b1=None, b2=None, S0=None, conv_in=None, *, out_dtype=torch.float32, seg_len: int | None = None,
                   o=None, S_final=None, conv_out=None, want_conv_out=True, ws=None, stream=None):
    """jb_prefill_from_x: the block from its layer input x (projections, generator, recurrence).
    Returns dict(o, S_final, conv_out)."""
    shape = _proj_shape(x, Wq, Wv, Wa, seg_len, out_dtype)
    B, T, H, dk, dv = shape.B, shape.T, shape.H, shape.dk, shape.dv
    dev = x.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    if S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if conv_out is None and want_conv_out:
        conv_out = torch.empty((B, 3, H, dv), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = workspace(prefill_from_x_workspace_size(shape), dev)
    _check(_lib.jb_prefill_from_x(ctypes.byref(shape), _ptr(x), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wa), _ptr(ba),
                                  _ptr(Wb), _ptr(bb), _ptr(W1), _ptr(b1), _ptr(W2),
                                  _ptr(b2), _ptr(S0), _ptr(conv_in), _ptr(o), _ptr(S_final), _ptr(conv_out),
                                  _ptr(ws), ws.numel(), _stream(stream)))
    return dict(o=o, S_final=S_final, conv_out=conv_out)


def decode_step_from_x_workspace_size(shape: Shape) -> int:
    n = _SZ(0)
    _check(_lib.jb_decode_step_from_x_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def decode_step_from_x(S, cache, x_t, Wq, Wk, Wv, Wa, Wb, W1, W2, ba=None, bb=None, b1=None, b2=None, *,
                       out_dtype=torch.float32, S_out=None, cache_out=None, o=None, ws=None, stream=None):
    """jb_decode_step_from_x: one decode step from the layer input x_t [B,D].  In place on S
    and cache unless S_out/cache_out are given.  Returns dict(o, S, cache)."""
    B, D = x_t.shape
    H = Wa.shape[0]
    dk, dv = Wq.shape[0] // H, Wv.shape[0] // H
    shape = make_shape(B, 1, H, dk, dv, D, JB_BF16, _DT[out_dtype])
    S_out = S if S_out is None else S_out
    cache_out = cache if cache_out is None else cache_out
    if o is None:
        o = torch.empty((B, H, dv), dtype=out_dtype, device=x_t.device)
    if ws is None:
        ws = workspace(decode_step_from_x_workspace_size(shape), x_t.device)
    _check(_lib.jb_decode_step_from_x(ctypes.byref(shape), _ptr(S), _ptr(S_out), _ptr(cache), _ptr(cache_out),
                                      _ptr(x_t), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wa), _ptr(ba), _ptr(Wb),
                                      _ptr(bb), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), _ptr(o), _ptr(ws),
                                      ws.numel(), _stream(stream)))
    return dict(o=o, S=S_out, cache=cache_out)


def prefill_static_workspace_size(shape: Shape) -> int:
    n = _SZ(0)
    _check(_lib.jb_prefill_static_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def prefill_static(q, k, v, alpha, beta, wq, wk, wv, S0=None, cache_q=None, cache_k=None, cache_v=None, *,
                   out_dtype=torch.float32, seg_len: int | None = None, o=None, S_final=None,
                   want_cache_out=True, ws=None, stream=None, d_model: int = 128):
    """jb_prefill_static: the static-conv block.  q,k [B,T,H,dk], v [B,T,H,dv] (bf16), alpha,beta
    [B,T,H] f32, weights wq,wk [H*dk,4], wv [H*dv,4] f32, caches [B,3,H,d] (all three or none).
    Returns dict(o, S_final, cache_q, cache_k, cache_v)."""
    B, T, H, dk = q.shape
    dv = v.shape[3]
    shape = make_shape(B, T, H, dk, dv, d_model, _io_code(q), _DT[out_dtype],
                       flag_segment(seg_len) if seg_len else 0)
    dev = q.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    if S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    outs = [None, None, None]
    if want_cache_out:
        outs = [torch.empty((B, 3, H, d), dtype=q.dtype, device=dev) for d in (dk, dk, dv)]
    need = prefill_static_workspace_size(shape)
    if ws is None and need > 0:
        ws = workspace(need, dev)
    _check(_lib.jb_prefill_static(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                  _ptr(wq), _ptr(wk), _ptr(wv), _ptr(S0), _ptr(cache_q), _ptr(cache_k),
                                  _ptr(cache_v), _ptr(o), _ptr(S_final), _ptr(outs[0]), _ptr(outs[1]),
                                  _ptr(outs[2]), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return dict(o=o, S_final=S_final, cache_q=outs[0], cache_k=outs[1], cache_v=outs[2])


def decode_step_static(S, cache_q, cache_k, cache_v, q_t, k_t, v_t, alpha_t, beta_t, wq, wk, wv, *,
                       out_dtype=torch.float32, S_out=None, cache_q_out=None, cache_k_out=None,
                       cache_v_out=None, o=None, stream=None, d_model: int = 128):
    """jb_decode_step_static: one decode step of the static-conv block.  In place on S and the
    caches unless the *_out tensors are given.  Returns dict(o, S, cache_q, cache_k, cache_v)."""
    B, H, dk = q_t.shape
    dv = v_t.shape[2]
    shape = make_shape(B, 1, H, dk, dv, d_model, _io_code(q_t), _DT[out_dtype])
    S_out = S if S_out is None else S_out
    cq = cache_q if cache_q_out is None else cache_q_out
    ck = cache_k if cache_k_out is None else cache_k_out
    cv = cache_v if cache_v_out is None else cache_v_out
    if o is None:
        o = torch.empty((B, H, dv), dtype=out_dtype, device=q_t.device)
    _check(_lib.jb_decode_step_static(ctypes.byref(shape), _ptr(S), _ptr(S_out), _ptr(cache_q), _ptr(cache_k),
                                      _ptr(cache_v), _ptr(cq), _ptr(ck), _ptr(cv), _ptr(q_t), _ptr(k_t),
                                      _ptr(v_t), _ptr(alpha_t), _ptr(beta_t), _ptr(wq), _ptr(wk), _ptr(wv),
                                      _ptr(o), _stream(stream)))
    return dict(o=o, S=S_out, cache_q=cq, cache_k=ck, cache_v=cv)


def prefill_varlen_workspace_size(shape: Shape, total_tokens: int) -> int:
    n = _SZ(0)
    _check(_lib.jb_prefill_varlen_workspace_size(ctypes.byref(shape), int(total_tokens), ctypes.byref(n)))
    return n.value


def prefill_varlen(cu_seqlens, x, q, k, v, alpha, beta, W1, W2, b1=None, b2=None, S0=None, conv_in=None, *,
                   max_seqlen: int | None = None, out_dtype=torch.float32, seg_len: int | None = None, o=None,
                   S_final=None, conv_out=None, want_conv_out=True, ws=None, stream=None):
    """jb_prefill_varlen: B packed sequences.  cu_seqlens int32 [B+1] (device; its host copy is
    read once for the longest length unless max_seqlen is given), x [total,D], q,k [total,H,dk],
    v [total,H,dv], alpha,beta [total,H].  Returns dict(o, S_final, conv_out) with per-sequence
    S_final [B,H,dk,dv] and conv_out [B,3,H,dv]."""
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    B = cu_seqlens.numel() - 1
    total, D = x.shape
    H, dk = q.shape[1], q.shape[2]
    dv = v.shape[2]
    if max_seqlen is None:
        lens = cu_seqlens.cpu().diff()
        max_seqlen = int(lens.max()) if B > 0 else 0
    shape = make_shape(B, max_seqlen, H, dk, dv, D, _io_code(x), _DT[out_dtype],
                       flag_segment(seg_len) if seg_len else 0)
    dev = x.device
    if o is None:
        o = torch.empty((total, H, dv), dtype=out_dtype, device=dev)
    if S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if conv_out is None and want_conv_out:
        conv_out = torch.empty((B, 3, H, dv), dtype=x.dtype, device=dev)
    need = prefill_varlen_workspace_size(shape, total)
    if ws is None:
        ws = workspace(need, dev)
    _check(_lib.jb_prefill_varlen(ctypes.byref(shape), total, _ptr(cu_seqlens), _ptr(x), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(alpha), _ptr(beta), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), _ptr(S0),
                                  _ptr(conv_in), _ptr(o), _ptr(S_final), _ptr(conv_out), _ptr(ws), ws.numel(),
                                  _stream(stream)))
    return dict(o=o, S_final=S_final, conv_out=conv_out)


def backward_workspace_size(shape: Shape) -> int:
    n = _SZ(0)
    _check(_lib.jb_backward_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def backward(x, q, k, v, alpha, beta, W1, W2, dout, b1=None, b2=None, S0=None, conv_in=None, dS_final=None,
             dconv_out=None, *, ws=None, stream=None):
    """jb_backward: gradients of jb_prefill.  Returns a dict of float32 tensors dx, dq, dk, dv,
    dalpha, dbeta, dW1, db1, dW2, db2, dS0, dconv_in."""
    B, T, D = x.shape
    H, dk = q.shape[2], q.shape[3]
    dv = v.shape[3]
    shape = make_shape(B, T, H, dk, dv, D, _io_code(x), JB_F32)
    dev = x.device
    f = lambda *sz: torch.empty(sz, dtype=torch.float32, device=dev)
    out = dict(dx=f(B, T, D), dq=f(B, T, H, dk), dk=f(B, T, H, dk), dv=f(B, T, H, dv), dalpha=f(B, T, H),
               dbeta=f(B, T, H), dW1=f(32, D), db1=f(32), dW2=f(4 * H, 32), db2=f(4 * H), dS0=f(B, H, dk, dv),
               dconv_in=f(B, 3, H, dv))
    if ws is None:
        ws = workspace(backward_workspace_size(shape), dev)
    _check(_lib.jb_backward(ctypes.byref(shape), _ptr(x), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                            _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), _ptr(S0), _ptr(conv_in), _ptr(dout),
                            _ptr(dS_final), _ptr(dconv_out),
                            *[_ptr(out[n]) for n in ("dx", "dq", "dk", "dv", "dalpha", "dbeta", "dW1", "db1", "dW2",
                                                     "db2", "dS0", "dconv_in")],
                            _ptr(ws), ws.numel(), _stream(stream)))
    return out
