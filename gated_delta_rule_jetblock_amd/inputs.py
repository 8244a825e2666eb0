"""Seeded synthetic inputs for the JetBlock token mixer.

This module only draws random numbers.  It holds none of the block's
arithmetic, so both the GPU library's tests and the fp64 oracle can take their
inputs from it.

Workload shapes follow the Jet-Nemotron pages: the xugj520 blog (section 2.2)
lists Q/K dimension 96 (2B) / 128 (4B), V dimension 256, 12 (2B) / 16 (4B)
heads, conv kernel size 4 and generator hidden width 32; model widths 1536
(2B, Qwen2.5-1.5B base) and 2048 (4B, Qwen2.5-3B base) follow from the base
models named in the csdn translation, section 3.1.  The throughput setting of
the pages is a 64K-token context, and 256K for the long-context figures.

Distributions (N(m, s): mean m, standard deviation s), drawn in this order from
one torch generator seeded per workload:
    x ~ N(0,1); q ~ N(0,1); k ~ N(0,1); v ~ N(0,1);
    alpha = sigmoid(N(3,1)); beta = sigmoid(N(0,1));
    W1 ~ N(0,0.02); W2 ~ N(0,0.02)   (no biases)
and for decode workloads, after those: the state S ~ N(0,0.1) and the conv
cache ~ N(0,1), then every step's (x, q, k, v, alpha, beta) in step order.
Packed batches (packed_prefill_inputs) draw one sequence of the total length
with the recipe above and cut it at the given lengths; serving mixes draw the
lengths uniformly from a range (request_lengths).
The static-conv block's weights (static_conv_inputs) are drawn from a generator
of their own: wq, wk, wv ~ U(-1/2, 1/2), the usual default initialisation of a
depthwise conv of size 4 (bound 1/sqrt(fan-in)), and caches ~ N(0,1).
q and k are handed to the block raw: normalising them is the block's job.
Tensors of the I/O dtype are drawn in float32 and rounded to nearest-even when
the I/O dtype is bfloat16; alpha, beta and the state are always float32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Shape:
    """Block shape: B sequences, T tokens, H heads, dk/dv head dims, d_model."""
    B: int
    T: int
    H: int
    dk: int
    dv: int
    d_model: int
    gen_hidden: int = 32
    taps: int = 4
    chunk: int = 64
    io_dtype: str = "bf16"      # x, q, k, v, W1, W2, conv cache: "bf16" or "f32"
    out_dtype: str = "f32"      # o: "f32" or "bf16"

    def with_(self, **kw) -> "Shape":
        return replace(self, **kw)


# Named workloads (seed 0 unless a test says otherwise).
TINY_F32 = Shape(B=1, T=256, H=2, dk=32, dv=64, d_model=128, io_dtype="f32")
B2_T4096 = Shape(B=1, T=4096, H=12, dk=96, dv=256, d_model=1536)
B2_T65536 = Shape(B=1, T=65536, H=12, dk=96, dv=256, d_model=1536)
B2_DECODE = Shape(B=256, T=1, H=12, dk=96, dv=256, d_model=1536)
B4_T262144 = Shape(B=1, T=262144, H=16, dk=128, dv=256, d_model=2048)
B4_DECODE = Shape(B=128, T=1, H=16, dk=128, dv=256, d_model=2048)
DECODE_STEPS = 128

WORKLOADS = {
    "tiny_f32_T256": TINY_F32,
    "jetblock2b_prefill_T4096": B2_T4096,
    "jetblock2b_prefill_T65536": B2_T65536,
    "jetblock2b_decode_B256": B2_DECODE,
    "jetblock4b_prefill_T262144": B4_T262144,
    "jetblock4b_decode_B128": B4_DECODE,
}


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(g, shape, mean, std, device, dtype):
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t if dtype == torch.float32 else t.to(dtype)


def prefill_inputs(shape: Shape, seed: int = 0, device="cpu", alpha_mean: float = 3.0,
                   beta_mean: float = 0.0):
    """Inputs of one prefill call: dict of tensors on `device`.

    alpha_mean / beta_mean shift the gate logits (3 and 0 for the named
    workloads; long-memory tests use larger alpha_mean and negative beta_mean).
    """
    s = shape
    io = torch_dtype(s.io_dtype)
    g = _gen(seed, device)
    x = _normal(g, (s.B, s.T, s.d_model), 0.0, 1.0, device, io)
    q = _normal(g, (s.B, s.T, s.H, s.dk), 0.0, 1.0, device, io)
    k = _normal(g, (s.B, s.T, s.H, s.dk), 0.0, 1.0, device, io)
    v = _normal(g, (s.B, s.T, s.H, s.dv), 0.0, 1.0, device, io)
    alpha = torch.sigmoid(_normal(g, (s.B, s.T, s.H), alpha_mean, 1.0, device, torch.float32))
    beta = torch.sigmoid(_normal(g, (s.B, s.T, s.H), beta_mean, 1.0, device, torch.float32))
    W1 = _normal(g, (s.gen_hidden, s.d_model), 0.0, 0.02, device, io)
    W2 = _normal(g, (s.H * s.taps, s.gen_hidden), 0.0, 0.02, device, io)
    return dict(x=x, q=q, k=k, v=v, alpha=alpha, beta=beta, W1=W1, W2=W2)


def state_inputs(shape: Shape, seed: int = 0, device="cpu", state_std: float = 0.1):
    """A seeded recurrent state S [B,H,dk,dv] f32 and conv cache [B,K-1,H,dv] (I/O dtype)."""
    s = shape
    g = _gen(seed + 7919, device)
    S = _normal(g, (s.B, s.H, s.dk, s.dv), 0.0, state_std, device, torch.float32)
    cache = _normal(g, (s.B, s.taps - 1, s.H, s.dv), 0.0, 1.0, device, torch_dtype(s.io_dtype))
    return dict(S=S, cache=cache)


def decode_inputs(shape: Shape, steps: int = DECODE_STEPS, seed: int = 0, device="cpu",
                  with_state: bool = True):
    """Inputs of `steps` decode steps for B sequences.

    Returns dict with W1, W2 (as for prefill), S [B,H,dk,dv] f32 and cache
    [B,K-1,H,dv] (when with_state), and per-step stacks x [steps,B,D],
    q,k [steps,B,H,dk], v [steps,B,H,dv], alpha, beta [steps,B,H].
    """
    s = shape
    io = torch_dtype(s.io_dtype)
    g = _gen(seed, device)
    W1 = _normal(g, (s.gen_hidden, s.d_model), 0.0, 0.02, device, io)
    W2 = _normal(g, (s.H * s.taps, s.gen_hidden), 0.0, 0.02, device, io)
    out = dict(W1=W1, W2=W2)
    if with_state:
        out["S"] = _normal(g, (s.B, s.H, s.dk, s.dv), 0.0, 0.1, device, torch.float32)
        out["cache"] = _normal(g, (s.B, s.taps - 1, s.H, s.dv), 0.0, 1.0, device, io)
    out["x"] = _normal(g, (steps, s.B, s.d_model), 0.0, 1.0, device, io)
    out["q"] = _normal(g, (steps, s.B, s.H, s.dk), 0.0, 1.0, device, io)
    out["k"] = _normal(g, (steps, s.B, s.H, s.dk), 0.0, 1.0, device, io)
    out["v"] = _normal(g, (steps, s.B, s.H, s.dv), 0.0, 1.0, device, io)
    out["alpha"] = torch.sigmoid(_normal(g, (steps, s.B, s.H), 3.0, 1.0, device, torch.float32))
    out["beta"] = torch.sigmoid(_normal(g, (steps, s.B, s.H), 0.0, 1.0, device, torch.float32))
    return out


def projection_inputs(shape: Shape, seed: int = 0, device="cpu", alpha_mean: float = 3.0,
                      beta_mean: float = 0.0):
    """Inputs of the block from its layer input: x [B,T,D] ~ N(0,1) and bf16 weights.

    Wq, Wk [H*dk, D], Wv [H*dv, D] ~ N(0, 1/D), so q, k, v come out ~ N(0, 1) like the
    direct-input workloads; Wa, Wb [H, D] ~ N(0, 1/D) with biases ba = alpha_mean,
    bb = beta_mean, so the gate logits are ~ N(mean, 1) as there; W1, W2 as for prefill.
    with_qkv_bias adds bq, bk, bv ~ N(0, 0.1).
    """
    s = shape
    io = torch.bfloat16
    g = _gen(seed, device)
    ws = 1.0 / math.sqrt(s.d_model)
    out = dict(
        x=_normal(g, (s.B, s.T, s.d_model), 0.0, 1.0, device, io),
        Wq=_normal(g, (s.H * s.dk, s.d_model), 0.0, ws, device, io),
        Wk=_normal(g, (s.H * s.dk, s.d_model), 0.0, ws, device, io),
        Wv=_normal(g, (s.H * s.dv, s.d_model), 0.0, ws, device, io),
        Wa=_normal(g, (s.H, s.d_model), 0.0, ws, device, io),
        Wb=_normal(g, (s.H, s.d_model), 0.0, ws, device, io),
        ba=torch.full((s.H,), alpha_mean, device=device).to(io),
        bb=torch.full((s.H,), beta_mean, device=device).to(io),
        W1=_normal(g, (s.gen_hidden, s.d_model), 0.0, 0.02, device, io),
        W2=_normal(g, (s.H * s.taps, s.gen_hidden), 0.0, 0.02, device, io),
    )
    return out


def static_conv_inputs(shape: Shape, seed: int = 0, device="cpu"):
    """Weights of the static-conv block, wq, wk [H*dk, 4] and wv [H*dv, 4] f32 ~ U(-1/2, 1/2),
    and raw-row caches cache_q, cache_k [B,3,H,dk], cache_v [B,3,H,dv] ~ N(0,1) (I/O dtype)."""
    s = shape
    io = torch_dtype(s.io_dtype)
    g = _gen(seed + 104729, device)

    def unif(rows):
        return torch.rand((rows, s.taps), generator=g, device=device, dtype=torch.float32) - 0.5

    out = dict(wq=unif(s.H * s.dk), wk=unif(s.H * s.dk), wv=unif(s.H * s.dv))
    out["cache_q"] = _normal(g, (s.B, s.taps - 1, s.H, s.dk), 0.0, 1.0, device, io)
    out["cache_k"] = _normal(g, (s.B, s.taps - 1, s.H, s.dk), 0.0, 1.0, device, io)
    out["cache_v"] = _normal(g, (s.B, s.taps - 1, s.H, s.dv), 0.0, 1.0, device, io)
    return out


def request_lengths(n: int, lo: int, hi: int, seed: int = 0) -> list[int]:
    """n sequence lengths drawn uniformly from [lo, hi] (a serving batch's length mix)."""
    g = _gen(seed + 31337, "cpu")
    return [int(t) for t in torch.randint(lo, hi + 1, (n,), generator=g)]


def packed_prefill_inputs(lengths, H: int, dk: int, dv: int, d_model: int, seed: int = 0, device="cpu",
                          io_dtype: str = "bf16"):
    """Inputs of a packed batch: sequences of the given lengths back to back.  Returns the
    prefill_inputs tensors without the batch axis (x [total,D], q,k [total,H,dk], v [total,H,dv],
    alpha,beta [total,H], W1, W2) and cu_seqlens int32 [len(lengths)+1]."""
    total = int(sum(lengths))
    shape = Shape(B=1, T=total, H=H, dk=dk, dv=dv, d_model=d_model, io_dtype=io_dtype)
    p = prefill_inputs(shape, seed=seed, device=device)
    out = {k: (v[0] if k not in ("W1", "W2") else v) for k, v in p.items()}
    cu = [0]
    for t in lengths:
        cu.append(cu[-1] + int(t))
    out["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=device)
    return out
