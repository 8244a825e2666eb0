"""GPU parity of the single-stage entry points and of the matrix-core placement.

Each stage is compared with the fp64 oracle (or, for the placement probe,
with an exact host product) through the C ABI.
"""
import numpy as np
import pytest
import torch

from helpers import rel_err, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def jb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_jetblock_amd import jetblock
    return jetblock


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_mfma_placement(jb, kind):
    """The operand placement all kernels assume reproduces an exact product
    (small integers are exact in fp16, bf16 and fp32)."""
    print(f"probe kind={kind}", flush=True)
    g = torch.Generator().manual_seed(kind)
    A = torch.randint(-4, 5, (16, 32), generator=g).float()
    B = torch.randint(-4, 5, (32, 16), generator=g).float()
    D = jb.probe_mfma(kind, A.cuda(), B.cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(D.cpu().numpy(), (A @ B).numpy())


@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("B,T,H,D", [(1, 5, 2, 128), (2, 70, 12, 1536), (3, 33, 16, 2048)])
def test_gen_taps(jb, oracle_mod, io, B, T, H, D):
    from gated_delta_rule_jetblock_amd import inputs
    print(f"gen_taps io={io} B={B} T={T} H={H} D={D}", flush=True)
    s = inputs.Shape(B=B, T=T, H=H, dk=32, dv=64, d_model=D, io_dtype="bf16" if io == torch.bfloat16 else "f32")
    p = inputs.prefill_inputs(s, seed=3)
    g = torch.Generator().manual_seed(5)
    b1 = (torch.randn(32, generator=g) * 0.5).to(io)
    b2 = (torch.randn(4 * H, generator=g) * 0.5).to(io)
    W1 = p["W1"] * 20  # wider pre-activation range so SiLU's curve matters
    taps = jb.gen_taps(p["x"].cuda(), W1.cuda(), p["W2"].cuda(), b1.cuda(), b2.cuda(), H=H)
    ref = oracle_mod.gen_taps(to_np(p["x"]), to_np(W1), to_np(p["W2"]), b1=to_np(b1), b2=to_np(b2), H=H)
    err = rel_err(taps, ref)
    assert err < (1e-4 if io == torch.bfloat16 else 1e-5), err


@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("with_cache", [False, True])
def test_gen_conv(jb, oracle_mod, io, with_cache):
    from gated_delta_rule_jetblock_amd import inputs
    print(f"gen_conv io={io} cache={with_cache}", flush=True)
    s = inputs.Shape(B=2, T=37, H=3, dk=32, dv=128, d_model=256, io_dtype="bf16" if io == torch.bfloat16 else "f32")
    p = inputs.prefill_inputs(s, seed=4)
    cache = inputs.state_inputs(s, seed=4)["cache"] if with_cache else None
    W1 = p["W1"] * 20
    taps, vc = jb.gen_conv(p["x"].cuda(), W1.cuda(), p["W2"].cuda(), p["v"].cuda(),
                           conv_in=None if cache is None else cache.cuda())
    rt = oracle_mod.gen_taps(to_np(p["x"]), to_np(W1), to_np(p["W2"]), H=3)
    rv = oracle_mod.conv(rt, to_np(p["v"]), to_np(cache))
    assert rel_err(taps, rt) < 1e-4
    assert rel_err(vc, rv) < 1e-4


@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("dk,T", [(32, 5), (96, 130), (128, 64), (64, 200)])
def test_prologue(jb, oracle_mod, io, dk, T):
    from gated_delta_rule_jetblock_amd import inputs
    print(f"prologue io={io} dk={dk} T={T}", flush=True)
    s = inputs.Shape(B=2, T=T, H=3, dk=dk, dv=64, d_model=128, io_dtype="bf16" if io == torch.bfloat16 else "f32")
    p = inputs.prefill_inputs(s, seed=6)
    qh, kh, g = jb.prologue(p["q"].cuda(), p["k"].cuda(), p["alpha"].cuda())
    assert rel_err(qh, oracle_mod.l2norm(to_np(p["q"]))) < 1e-6
    assert rel_err(kh, oracle_mod.l2norm(to_np(p["k"]))) < 1e-6
    # g: inclusive cumulative sum of ln(alpha) restarting every 64 tokens
    la = np.log(to_np(p["alpha"]).astype(np.float64))
    want = np.empty_like(la)
    for c0 in range(0, T, 64):
        want[:, c0:c0 + 64] = np.cumsum(la[:, c0:c0 + 64], axis=1)
    np.testing.assert_allclose(g.cpu().numpy(), want, rtol=1e-5, atol=1e-5)
