"""GPU parity of jb_decode_step against the fp64 oracle: the 2B decode workload
(B=256 sequences, 128 steps from a seeded state), the 4B decode shape, both
I/O dtypes, in-place state and cache, and prefill = decode loop."""
import numpy as np
import pytest
import torch

from helpers import TOL_BF16, TOL_F32, rel_err, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def jb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_jetblock_amd import jetblock
    return jetblock


def _decode_vs_oracle(jb, oracle_mod, shape, steps, sample_b, io_tol, seed=0, out_dtype=torch.float32):
    from gated_delta_rule_jetblock_amd import inputs
    d = inputs.decode_inputs(shape, steps=steps, seed=seed)
    S = d["S"].cuda().clone()
    cache = d["cache"].cuda().clone()
    W1, W2 = d["W1"].cuda(), d["W2"].cuda()
    dev = {k: d[k].cuda() for k in ("x", "q", "k", "v", "alpha", "beta")}
    outs = []
    for t in range(steps):
        r = jb.decode_step(S, cache, dev["x"][t], dev["q"][t], dev["k"][t], dev["v"][t], dev["alpha"][t],
                           dev["beta"][t], W1, W2, out_dtype=out_dtype)
        outs.append(r["o"].clone())
    torch.cuda.synchronize()
    # oracle on sampled sequences, step by step from the same seeded state
    bs = np.array(sample_b)
    So = to_np(d["S"])[bs]
    co = to_np(d["cache"])[bs]
    worst_o = 0.0
    for t in range(steps):
        ro = oracle_mod.decode_step(So, co, to_np(d["x"][t])[bs], to_np(d["q"][t])[bs], to_np(d["k"][t])[bs],
                                    to_np(d["v"][t])[bs], to_np(d["alpha"][t])[bs], to_np(d["beta"][t])[bs],
                                    to_np(d["W1"]), to_np(d["W2"]))
        worst_o = max(worst_o, rel_err(outs[t][bs], ro["o"]))
        So, co = ro["S"], ro["cache"]
    es = rel_err(S[bs], So)
    print(f"  decode B={shape.B} steps={steps} o_err={worst_o:.3e} S_err={es:.3e}", flush=True)
    assert worst_o < io_tol and es < io_tol, (worst_o, es)
    np.testing.assert_array_equal(to_np(cache)[bs], co)


def test_jetblock2b_decode_B256(jb, oracle_mod):
    """JetBlock 2B decode: B=256, 128 steps from S ~ N(0, 0.1), 3-row conv cache, bf16 inputs.
    The GPU runs all 256 sequences; the oracle checks 12 of them at every step."""
    from gated_delta_rule_jetblock_amd import inputs
    print("2B decode B=256 x 128", flush=True)
    _decode_vs_oracle(jb, oracle_mod, inputs.B2_DECODE, 128, [0, 1, 17, 63, 64, 100, 127, 128, 200, 254, 255, 77],
                      TOL_BF16)


def test_jetblock4b_decode_shape(jb, oracle_mod):
    from gated_delta_rule_jetblock_amd import inputs
    print("4B decode B=128 x 16", flush=True)
    _decode_vs_oracle(jb, oracle_mod, inputs.B4_DECODE, 16, [0, 5, 64, 127], TOL_BF16, seed=3)


@pytest.mark.parametrize("dk,dv", [(32, 64), (64, 128), (128, 64), (96, 128)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_decode_shapes(jb, oracle_mod, dk, dv, io):
    from gated_delta_rule_jetblock_amd import inputs
    print(f"decode dk={dk} dv={dv} io={io}", flush=True)
    s = inputs.Shape(B=5, T=1, H=3, dk=dk, dv=dv, d_model=256, io_dtype=io)
    _decode_vs_oracle(jb, oracle_mod, s, 6, [0, 2, 4], TOL_BF16 if io == "bf16" else TOL_F32, seed=dk)


def test_decode_bf16_output_rounding(jb):
    from gated_delta_rule_jetblock_amd import inputs
    s = inputs.Shape(B=4, T=1, H=2, dk=96, dv=256, d_model=256)
    d = inputs.decode_inputs(s, steps=1, seed=5)
    args = [d[k][0].cuda() for k in ("x", "q", "k", "v", "alpha", "beta")] + [d["W1"].cuda(), d["W2"].cuda()]
    S1, c1 = d["S"].cuda().clone(), d["cache"].cuda().clone()
    S2, c2 = d["S"].cuda().clone(), d["cache"].cuda().clone()
    r32 = jb.decode_step(S1, c1, *args)
    r16 = jb.decode_step(S2, c2, *args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(r16["o"].view(torch.int16), r32["o"].to(torch.bfloat16).view(torch.int16))
    assert torch.equal(S1, S2)


def test_prefill_equals_decode_loop(jb, oracle_mod):
    """T decode steps from (S0, cache) match one prefill of the same T tokens."""
    from gated_delta_rule_jetblock_amd import inputs
    s = inputs.Shape(B=2, T=70, H=2, dk=64, dv=128, d_model=256)
    p = inputs.prefill_inputs(s, seed=31)
    st = inputs.state_inputs(s, seed=31)
    dp = {k: v.cuda() for k, v in p.items()}
    r = jb.prefill(dp["x"], dp["q"], dp["k"], dp["v"], dp["alpha"], dp["beta"], dp["W1"], dp["W2"],
                   S0=st["S"].cuda(), conv_in=st["cache"].cuda())
    S = st["S"].cuda().clone()
    c = st["cache"].cuda().clone()
    outs = []
    for t in range(s.T):
        rr = jb.decode_step(S, c, dp["x"][:, t].contiguous(), dp["q"][:, t].contiguous(), dp["k"][:, t].contiguous(),
                            dp["v"][:, t].contiguous(), dp["alpha"][:, t].contiguous(), dp["beta"][:, t].contiguous(),
                            dp["W1"], dp["W2"])
        outs.append(rr["o"].clone())
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=1)
    assert rel_err(o, to_np(r["o"]).astype(np.float64)) < TOL_BF16
    assert rel_err(S, to_np(r["S_final"]).astype(np.float64)) < TOL_BF16
    assert torch.equal(c, r["conv_out"])


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_decode_update_with_given_taps(jb, oracle_mod, io):
    """jb_gen_taps followed by jb_decode_update equals jb_decode_step (and the oracle)."""
    from gated_delta_rule_jetblock_amd import inputs
    s = inputs.Shape(B=6, T=1, H=3, dk=64, dv=128, d_model=256, io_dtype=io)
    d = inputs.decode_inputs(s, steps=1, seed=17)
    g = torch.Generator().manual_seed(3)
    b1 = (torch.randn(32, generator=g) * 0.3).to(d["W1"].dtype).cuda()
    b2 = (torch.randn(12, generator=g) * 0.3).to(d["W1"].dtype).cuda()
    args = [d[k][0].cuda() for k in ("x", "q", "k", "v", "alpha", "beta")]
    W1, W2 = d["W1"].cuda(), d["W2"].cuda()
    S1, c1 = d["S"].cuda().clone(), d["cache"].cuda().clone()
    S2, c2 = d["S"].cuda().clone(), d["cache"].cuda().clone()
    r1 = jb.decode_step(S1, c1, *args, W1, W2, b1, b2)
    taps = jb.gen_taps(args[0].view(6, 1, 256), W1, W2, b1, b2, H=3)
    r2 = jb.decode_update(S2, c2, args[1], args[2], args[3], args[4], args[5], taps, d_model=256)
    torch.cuda.synchronize()
    ro = oracle_mod.decode_step(to_np(d["S"]), to_np(d["cache"]), *(to_np(a) for a in args), to_np(d["W1"]),
                                to_np(d["W2"]), b1=to_np(b1), b2=to_np(b2))
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    assert rel_err(r1["o"], ro["o"]) < tol and rel_err(S1, ro["S"]) < tol
    assert rel_err(r2["o"], ro["o"]) < tol and rel_err(S2, ro["S"]) < tol
    assert torch.equal(c1, c2)


@pytest.mark.parametrize("B,H,dk,dv", [(64, 12, 96, 256), (32, 16, 64, 128), (256, 20, 32, 64), (16, 5, 128, 256)])
def test_decode_head_groups(jb, oracle_mod, B, H, dk, dv):
    """jb_decode_step gives each workgroup one sequence and a group of its heads: groups
    of 3 (odd), 2, 10 (H = 20 split in two) and 1 head, against the oracle."""
    from gated_delta_rule_jetblock_amd import inputs
    print(f"decode groups B={B} H={H} dk={dk} dv={dv}", flush=True)
    s = inputs.Shape(B=B, T=1, H=H, dk=dk, dv=dv, d_model=512)
    _decode_vs_oracle(jb, oracle_mod, s, 3, [0, B // 2, B - 1], TOL_BF16, seed=B + H)
