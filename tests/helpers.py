"""Shared helpers for the parity tests: error metric, oracle calls on tensors."""
import numpy as np
import torch

# Tolerances: max|gpu - oracle| / max|oracle| per output tensor.
TOL_BF16 = 2e-3   # bf16 inputs, fp32 accumulation
TOL_F32 = 1e-5    # all-fp32 mode


def rel_err(gpu, ref) -> float:
    g = gpu.detach().float().cpu().numpy().astype(np.float64) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    denom = np.abs(r).max()
    return float(np.abs(g - r).max() / (denom if denom > 0 else 1.0))


def to_np(t):
    """Exact float32 numpy copy of a tensor (bf16 widens exactly)."""
    return None if t is None else t.detach().float().cpu().numpy()


def tol_for(io_dtype) -> float:
    return TOL_F32 if io_dtype == torch.float32 else TOL_BF16


def oracle_prefill(oracle, p, S0=None, conv_in=None, heads=None, tokens=None, nthreads=None):
    """Run the oracle on inputs p (dict of tensors), optionally on a subset of heads
    and a prefix of tokens.  Returns the oracle's dict."""
    def sl(t, axis_h=2):
        a = to_np(t)
        if tokens is not None:
            a = a[:, :tokens]
        if heads is not None:
            a = a[:, :, heads] if a.ndim >= 3 else a
        return np.ascontiguousarray(a)
    x = to_np(p["x"])
    if tokens is not None:
        x = x[:, :tokens]
    W2 = to_np(p["W2"])
    if heads is not None:
        rows = np.concatenate([np.arange(h * 4, h * 4 + 4) for h in heads])
        W2 = W2[rows]
    s0 = to_np(S0)
    ci = to_np(conv_in)
    if heads is not None:
        s0 = None if s0 is None else np.ascontiguousarray(s0[:, heads])
        ci = None if ci is None else np.ascontiguousarray(ci[:, :, heads])
    return oracle.prefill(np.ascontiguousarray(x), sl(p["q"]), sl(p["k"]), sl(p["v"]), sl(p["alpha"]),
                          sl(p["beta"]), to_np(p["W1"]), np.ascontiguousarray(W2), S0=s0, conv_in=ci,
                          nthreads=nthreads)


def to_dev(p, device="cuda"):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
