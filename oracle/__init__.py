"""fp64 CPU oracle for the JetBlock token mixer (ctypes wrapper over jbo.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing on the product path imports it,
and it imports nothing from the product package.

What it computes is stated in jbo.c: the Jet-Nemotron paper's JetBlock
(csdn translation, section 2.4; kernel size 4 and generator hidden 32 from the
xugj520 blog, section 2.2) with the Gated DeltaNet recurrence
S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v'_t k_t^T, o_t = S_t q_t, one token
at a time in double precision.  Every function here only marshals numpy
arrays; the arithmetic is in jbo.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "jbo.c")
_LIB = os.path.join(_HERE, "libjbo.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile jbo.c into libjbo.so with gcc (plain C, -O2, pthreads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_int64
        _lib.jbo_prefill.argtypes = [I] * 8 + [P] * 16 + [I]
        _lib.jbo_prefill.restype = I
        _lib.jbo_decode_step.argtypes = [I] * 7 + [P] * 15 + [I]
        _lib.jbo_decode_step.restype = I
        _lib.jbo_gen_taps.argtypes = [L, I, I, I, I, P, P, P, P, P, P, I]
        _lib.jbo_gen_taps.restype = I
        _lib.jbo_conv.argtypes = [I, I, I, I, I, P, P, P, P]
        _lib.jbo_conv.restype = I
        _lib.jbo_l2norm.argtypes = [L, I, P, P]
        _lib.jbo_l2norm.restype = I
        _lib.jbo_project.argtypes = [L, I, I, I, I] + [P] * 16 + [I]
        _lib.jbo_prefill_static.argtypes = [I] * 6 + [P] * 17 + [I]
        _lib.jbo_prefill_static.restype = I
        _lib.jbo_project.restype = I
        _lib.jbo_backward.argtypes = [I] * 8 + [P] * 27 + [I]
        _lib.jbo_backward.restype = I
        _lib.jbo_bf16_round.argtypes = [ctypes.c_double]
        _lib.jbo_bf16_round.restype = ctypes.c_double
    return _lib


def _f32(a):
    """Exact float32 copy of an input array (None passes through)."""
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def prefill(x, q, k, v, alpha, beta, W1, W2, b1=None, b2=None, S0=None, conv_in=None,
            K: int = 4, nthreads: int | None = None, want_taps: bool = False):
    """Run the block over x [B,T,D], q,k [B,T,H,dk], v [B,T,H,dv], alpha,beta [B,T,H].

    Returns dict(o [B,T,H,dv] f64, S_final [B,H,dk,dv] f64, conv_out [B,K-1,H,dv] f32,
    taps [B,T,H,K] f64 when want_taps).
    """
    x, q, k, v = _f32(x), _f32(q), _f32(k), _f32(v)
    alpha, beta, W1, W2 = _f32(alpha), _f32(beta), _f32(W1), _f32(W2)
    b1, b2, S0, conv_in = _f32(b1), _f32(b2), _f32(S0), _f32(conv_in)
    B, T, D = x.shape
    H, dk = q.shape[2], q.shape[3]
    dv = v.shape[3]
    G = W1.shape[0]
    assert q.shape == (B, T, H, dk) and k.shape == (B, T, H, dk)
    assert v.shape == (B, T, H, dv) and alpha.shape == (B, T, H) and beta.shape == (B, T, H)
    assert W1.shape == (G, D) and W2.shape == (H * K, G)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    if conv_in is not None:
        assert conv_in.shape == (B, K - 1, H, dv)
    o = np.empty((B, T, H, dv), np.float64)
    S = np.empty((B, H, dk, dv), np.float64)
    cout = np.empty((B, K - 1, H, dv), np.float32)
    taps = np.empty((B, T, H, K), np.float64) if want_taps else None
    rc = _load().jbo_prefill(B, T, H, dk, dv, D, G, K, _p(x), _p(q), _p(k), _p(v),
                             _p(alpha), _p(beta), _p(W1), _p(b1), _p(W2), _p(b2),
                             _p(S0), _p(conv_in), _p(o), _p(S), _p(cout), _p(taps),
                             nthreads or default_threads())
    if rc != 0:
        raise ValueError("jbo_prefill rejected its arguments")
    out = dict(o=o, S_final=S, conv_out=cout)
    if want_taps:
        out["taps"] = taps
    return out


def decode_step(S, cache, x_t, q_t, k_t, v_t, alpha_t, beta_t, W1, W2, b1=None, b2=None,
                K: int = 4, nthreads: int | None = None):
    """One token for B sequences.  Returns dict(o [B,H,dv], S [B,H,dk,dv], cache)."""
    S, cache = _f32(S), _f32(cache)
    x_t, q_t, k_t, v_t = _f32(x_t), _f32(q_t), _f32(k_t), _f32(v_t)
    alpha_t, beta_t, W1, W2, b1, b2 = (_f32(a) for a in (alpha_t, beta_t, W1, W2, b1, b2))
    B, D = x_t.shape
    H, dk = q_t.shape[1], q_t.shape[2]
    dv = v_t.shape[2]
    G = W1.shape[0]
    assert S.shape == (B, H, dk, dv) and cache.shape == (B, K - 1, H, dv)
    o = np.empty((B, H, dv), np.float64)
    S2 = np.empty((B, H, dk, dv), np.float64)
    c2 = np.empty((B, K - 1, H, dv), np.float32)
    rc = _load().jbo_decode_step(B, H, dk, dv, D, G, K, _p(S), _p(cache), _p(x_t), _p(q_t),
                                 _p(k_t), _p(v_t), _p(alpha_t), _p(beta_t), _p(W1), _p(b1),
                                 _p(W2), _p(b2), _p(o), _p(S2), _p(c2),
                                 nthreads or default_threads())
    if rc != 0:
        raise ValueError("jbo_decode_step rejected its arguments")
    return dict(o=o, S=S2, cache=c2)


def gen_taps(x, W1, W2, b1=None, b2=None, H: int | None = None, K: int = 4,
             nthreads: int | None = None):
    """Kernel generator on rows of x [..., D] -> taps [..., H, K] (f64)."""
    x = _f32(x)
    W1, W2, b1, b2 = _f32(W1), _f32(W2), _f32(b1), _f32(b2)
    D = x.shape[-1]
    n = int(np.prod(x.shape[:-1]))
    G = W1.shape[0]
    if H is None:
        H = W2.shape[0] // K
    taps = np.empty(x.shape[:-1] + (H, K), np.float64)
    rc = _load().jbo_gen_taps(n, D, G, H, K, _p(x), _p(W1), _p(b1), _p(W2), _p(b2), _p(taps),
                              nthreads or default_threads())
    if rc != 0:
        raise ValueError("jbo_gen_taps rejected its arguments")
    return taps


def conv(taps, v, conv_in=None):
    """Dynamic causal conv: taps [B,T,H,K] f64, v [B,T,H,dv] -> v' [B,T,H,dv] f64."""
    taps = np.ascontiguousarray(np.asarray(taps, np.float64))
    v, conv_in = _f32(v), _f32(conv_in)
    B, T, H, dv = v.shape
    K = taps.shape[-1]
    out = np.empty((B, T, H, dv), np.float64)
    rc = _load().jbo_conv(B, T, H, dv, K, _p(taps), _p(v), _p(conv_in), _p(out))
    if rc != 0:
        raise ValueError("jbo_conv rejected its arguments")
    return out


def l2norm(x):
    """Row-wise x * (sum x^2 + 1e-6)^(-1/2) along the last axis (f64)."""
    x = _f32(x)
    d = x.shape[-1]
    out = np.empty(x.shape, np.float64)
    rc = _load().jbo_l2norm(int(x.size // d), d, _p(x), _p(out))
    if rc != 0:
        raise ValueError("jbo_l2norm rejected its arguments")
    return out


def bf16_round(value: float) -> float:
    """Nearest bf16 of a double, ties to even (jbo_bf16_round)."""
    return _load().jbo_bf16_round(float(value))


def project(x, Wq, Wk, Wv, Wa, Wb, bq=None, bk=None, bv=None, ba=None, bb=None,
            nthreads: int | None = None):
    """The input projections of the block (jbo_project) for x [B,T,D]:
    Wq, Wk [H*dk, D], Wv [H*dv, D], Wa, Wb [H, D], biases optional.

    Returns dict(q, k [B,T,H,dk], v [B,T,H,dv] float32 holding bf16 values,
    alpha, beta [B,T,H] float64)."""
    x = _f32(x)
    Wq, Wk, Wv, Wa, Wb = _f32(Wq), _f32(Wk), _f32(Wv), _f32(Wa), _f32(Wb)
    bq, bk, bv, ba, bb = _f32(bq), _f32(bk), _f32(bv), _f32(ba), _f32(bb)
    B, T, D = x.shape
    H = Wa.shape[0]
    dk = Wq.shape[0] // H
    dv = Wv.shape[0] // H
    assert Wq.shape == (H * dk, D) and Wk.shape == (H * dk, D) and Wv.shape == (H * dv, D)
    assert Wa.shape == (H, D) and Wb.shape == (H, D)
    n = B * T
    q = np.empty((B, T, H, dk), np.float32)
    k = np.empty((B, T, H, dk), np.float32)
    v = np.empty((B, T, H, dv), np.float32)
    alpha = np.empty((B, T, H), np.float64)
    beta = np.empty((B, T, H), np.float64)
    rc = _load().jbo_project(n, D, H, dk, dv, _p(x), _p(Wq), _p(bq), _p(Wk), _p(bk), _p(Wv), _p(bv),
                             _p(Wa), _p(ba), _p(Wb), _p(bb), _p(q), _p(k), _p(v), _p(alpha), _p(beta),
                             nthreads or default_threads())
    if rc != 0:
        raise ValueError("jbo_project rejected its arguments")
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta)


def prefill_from_x(x, Wq, Wk, Wv, Wa, Wb, W1, W2, bq=None, bk=None, bv=None, ba=None, bb=None,
                   b1=None, b2=None, S0=None, conv_in=None, nthreads: int | None = None):
    """The block from its input x: project() and then prefill().  The gates
    cross into the block as float32, its boundary type; q, k, v as the bf16
    values project() returns."""
    pr = project(x, Wq, Wk, Wv, Wa, Wb, bq, bk, bv, ba, bb, nthreads)
    r = prefill(x, pr["q"], pr["k"], pr["v"], pr["alpha"].astype(np.float32), pr["beta"].astype(np.float32),
                W1, W2, b1=b1, b2=b2, S0=S0, conv_in=conv_in, nthreads=nthreads)
    r["proj"] = pr
    return r


def prefill_static(q, k, v, alpha, beta, wq, wk, wv, S0=None, cache_q=None, cache_k=None, cache_v=None,
                   nthreads: int | None = None):
    """The static-conv Gated DeltaNet block (jbo_prefill_static): per-channel causal convs of
    size K with fixed weights wq, wk [H*dk, K], wv [H*dv, K] on q, k, v, then the recurrence.

    Returns dict(o [B,T,H,dv] f64, S_final f64, cache_q, cache_k, cache_v [B,K-1,H,d] f32)."""
    q, k, v, alpha, beta = _f32(q), _f32(k), _f32(v), _f32(alpha), _f32(beta)
    wq, wk, wv, S0 = _f32(wq), _f32(wk), _f32(wv), _f32(S0)
    cache_q, cache_k, cache_v = _f32(cache_q), _f32(cache_k), _f32(cache_v)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    K = wq.shape[1]
    assert wq.shape == (H * dk, K) and wk.shape == (H * dk, K) and wv.shape == (H * dv, K)
    o = np.empty((B, T, H, dv), np.float64)
    S = np.empty((B, H, dk, dv), np.float64)
    cq = np.empty((B, K - 1, H, dk), np.float32)
    ck = np.empty((B, K - 1, H, dk), np.float32)
    cv = np.empty((B, K - 1, H, dv), np.float32)
    rc = _load().jbo_prefill_static(B, T, H, dk, dv, K, _p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(wq),
                                    _p(wk), _p(wv), _p(S0), _p(cache_q), _p(cache_k), _p(cache_v), _p(o), _p(S),
                                    _p(cq), _p(ck), _p(cv), nthreads or default_threads())
    if rc != 0:
        raise ValueError("jbo_prefill_static rejected its arguments")
    return dict(o=o, S_final=S, cache_q=cq, cache_k=ck, cache_v=cv)


def decode_step_static(S, cache_q, cache_k, cache_v, q_t, k_t, v_t, alpha_t, beta_t, wq, wk, wv,
                       nthreads: int | None = None):
    """One decode step of the static-conv block (prefill_static with T = 1); q_t, k_t [B,H,dk],
    v_t [B,H,dv], alpha_t, beta_t [B,H].  Returns dict(o [B,H,dv], S, cache_q, cache_k, cache_v)."""
    r = prefill_static(np.asarray(q_t)[:, None], np.asarray(k_t)[:, None], np.asarray(v_t)[:, None],
                       np.asarray(alpha_t)[:, None], np.asarray(beta_t)[:, None], wq, wk, wv, S0=S,
                       cache_q=cache_q, cache_k=cache_k, cache_v=cache_v, nthreads=nthreads)
    return dict(o=r["o"][:, 0], S=r["S_final"], cache_q=r["cache_q"], cache_k=r["cache_k"], cache_v=r["cache_v"])


def backward(x, q, k, v, alpha, beta, W1, W2, dout, b1=None, b2=None, S0=None, conv_in=None, dS_final=None,
             dconv_out=None, nthreads: int | None = None):
    """Reverse-mode gradient of prefill (jbo_backward) for the output gradients dout [B,T,H,dv],
    dS_final [B,H,dk,dv] and dconv_out [B,K-1,H,dv] (both nullable).  Returns a dict of f64
    arrays: dx, dq, dk, dv, dalpha, dbeta, dW1, db1, dW2, db2, dS0, dconv_in (the last two are
    gradients with respect to the zeros used when S0 / conv_in are None)."""
    x, q, k, v, alpha, beta = _f32(x), _f32(q), _f32(k), _f32(v), _f32(alpha), _f32(beta)
    W1, W2, b1, b2 = _f32(W1), _f32(W2), _f32(b1), _f32(b2)
    S0, conv_in, dout, dS_final, dconv_out = _f32(S0), _f32(conv_in), _f32(dout), _f32(dS_final), _f32(dconv_out)
    B, T, D = x.shape
    H, dk = q.shape[2], q.shape[3]
    dv = v.shape[3]
    G = W1.shape[0]
    K = W2.shape[0] // H
    out = dict(dx=np.empty((B, T, D)), dq=np.empty((B, T, H, dk)), dk=np.empty((B, T, H, dk)),
               dv=np.empty((B, T, H, dv)), dalpha=np.empty((B, T, H)), dbeta=np.empty((B, T, H)),
               dW1=np.empty((G, D)), db1=np.empty(G), dW2=np.empty((H * K, G)), db2=np.empty(H * K),
               dS0=np.empty((B, H, dk, dv)), dconv_in=np.empty((B, K - 1, H, dv)))
    rc = _load().jbo_backward(B, T, H, dk, dv, D, G, K, _p(x), _p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(W1),
                              _p(b1), _p(W2), _p(b2), _p(S0), _p(conv_in), _p(dout), _p(dS_final), _p(dconv_out),
                              *[_p(out[n]) for n in ("dx", "dq", "dk", "dv", "dalpha", "dbeta", "dW1", "db1", "dW2",
                                                     "db2", "dS0", "dconv_in")], nthreads or default_threads())
    if rc != 0:
        raise ValueError("jbo_backward rejected its arguments")
    return out
