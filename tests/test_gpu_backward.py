"""GPU parity of the backward pass (jb_backward) against the fp64 oracle's reverse-mode
gradient (jbo_backward): every gradient tensor within the tolerance below, on ragged chunk
counts, with and without initial state and cache, and at the 2B head shape."""
import numpy as np
import pytest
import torch

from helpers import rel_err, to_np

pytestmark = pytest.mark.gpu

from gated_delta_rule_jetblock_amd.inputs import Shape, prefill_inputs, state_inputs

# bf16 inputs, fp16 matrix-core operands with fp32 accumulation (as the forward pass);
# gradients pass through about twice the operations of the forward pass, so the bar is
# twice the forward one
TOL = 4e-3
NAMES = ("dx", "dq", "dk", "dv", "dalpha", "dbeta", "dW1", "db1", "dW2", "db2", "dS0", "dconv_in")


@pytest.fixture(scope="module")
def jb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_jetblock_amd import jetblock
    return jetblock


def _case(shape, seed, with_state=True, with_grads=True):
    p = prefill_inputs(shape, seed=seed)
    g = torch.Generator().manual_seed(seed + 17)
    d = dict(p)
    if with_state:
        st = state_inputs(shape, seed=seed)
        d["S0"], d["conv_in"] = st["S"], st["cache"]
    d["dout"] = torch.randn((shape.B, shape.T, shape.H, shape.dv), generator=g)
    if with_grads:
        d["dS_final"] = torch.randn((shape.B, shape.H, shape.dk, shape.dv), generator=g) * 0.1
        d["dconv_out"] = torch.randn((shape.B, 3, shape.H, shape.dv), generator=g)
    return d


def _run(jb, oracle_mod, shape, seed, with_state=True, with_grads=True, nthreads=None):
    d = _case(shape, seed, with_state, with_grads)
    g = {k: v.cuda() for k, v in d.items()}
    r = jb.backward(g["x"], g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["W1"], g["W2"], g["dout"],
                    S0=g.get("S0"), conv_in=g.get("conv_in"), dS_final=g.get("dS_final"),
                    dconv_out=g.get("dconv_out"))
    torch.cuda.synchronize()
    ref = oracle_mod.backward(to_np(d["x"]), to_np(d["q"]), to_np(d["k"]), to_np(d["v"]), to_np(d["alpha"]),
                              to_np(d["beta"]), to_np(d["W1"]), to_np(d["W2"]), to_np(d["dout"]),
                              S0=to_np(d.get("S0")), conv_in=to_np(d.get("conv_in")),
                              dS_final=to_np(d.get("dS_final")), dconv_out=to_np(d.get("dconv_out")),
                              nthreads=nthreads)
    errs = {n: rel_err(r[n], ref[n]) for n in NAMES}
    print("  " + "  ".join(f"{n} {e:.1e}" for n, e in errs.items()), flush=True)
    return errs


@pytest.mark.parametrize("B,T,H,dk,dv,D,state,grads", [
    (2, 200, 2, 32, 64, 128, True, True),      # 3 chunks + a ragged tail
    (1, 64, 2, 32, 64, 128, False, False),     # one full chunk, zero state, only dO
    (2, 1, 1, 32, 64, 128, True, True),        # a single token
    (1, 300, 3, 64, 128, 256, True, True),
    (1, 260, 2, 96, 256, 256, True, True),
    (1, 130, 1, 128, 256, 128, True, True),
])
def test_backward_vs_oracle(jb, oracle_mod, B, T, H, dk, dv, D, state, grads):
    print(f"[backward B={B} T={T} H={H} dk={dk} dv={dv} D={D} state={state} grads={grads}]", flush=True)
    errs = _run(jb, oracle_mod, Shape(B=B, T=T, H=H, dk=dk, dv=dv, d_model=D), seed=T + dk, with_state=state,
                with_grads=grads)
    bad = {n: e for n, e in errs.items() if not e < TOL}
    assert not bad, bad


def test_backward_jetblock2b_T1024(jb, oracle_mod):
    """The 2B head shape (H = 12, dk = 96, dv = 256, d_model = 1536) over 1,024 tokens."""
    print("[backward 2B T=1024]", flush=True)
    errs = _run(jb, oracle_mod, Shape(B=1, T=1024, H=12, dk=96, dv=256, d_model=1536), seed=5)
    bad = {n: e for n, e in errs.items() if not e < TOL}
    assert not bad, bad


def test_backward_training_shape_B16_T4096(jb, oracle_mod):
    """The training shape the bench times: B=16 sequences x T=4,096 tokens at the 2B head
    shape (H=12, dk=96, dv=256, d_model=1536), 1,024 chunks per head in all, with initial
    states and conv caches and every output gradient; every gradient tensor against the
    oracle over all sixteen sequences and twelve heads."""
    print("[backward B=16 T=4096 2B heads]", flush=True)
    errs = _run(jb, oracle_mod, Shape(B=16, T=4096, H=12, dk=96, dv=256, d_model=1536), seed=31)
    assert max(errs.values()) < TOL, errs
