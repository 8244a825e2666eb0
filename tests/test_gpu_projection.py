"""GPU parity of the block from its layer input x (jb_project, jb_prefill_from_x) against
the fp64 oracle: q, k, v within one bf16 step (plus the fp32 summation bound) of the
oracle's rounding of the exact sum, the gates and taps in fp32 precision, and the whole
block within the bf16-input bar."""
import numpy as np
import pytest
import torch

from helpers import TOL_BF16, rel_err, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def jb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_jetblock_amd import jetblock
    return jetblock


_W = ("Wq", "Wk", "Wv", "Wa", "Wb", "W1", "W2")
_B = ("ba", "bb")


def _oracle_args(p):
    return dict({k: to_np(p[k]) for k in ("x",) + _W}, **{k: to_np(p[k]) for k in _B if k in p})


def _bf16_spacing(v):
    m = np.abs(np.asarray(v, np.float64))
    return np.exp2(np.floor(np.log2(np.where(m > 0, m, 1.0))) - 7)


def _check_projections(r, ref, p, what):
    """The GPU sums D products in fp32 and rounds once to bf16; the oracle rounds the exact
    sum.  Per element the two may differ by one bf16 step at the larger of them plus the fp32
    summation bound D 2^-24 sum_i |w_i x_i| (which dominates where the sum nearly cancels)."""
    x = np.abs(to_np(p["x"]).astype(np.float64)).reshape(-1, p["x"].shape[-1])
    D = x.shape[1]
    for key, w in (("q", "Wq"), ("k", "Wk"), ("v", "Wv")):
        g = to_np(r[key]).astype(np.float64).reshape(x.shape[0], -1)
        ref_k = np.asarray(ref[key], np.float64).reshape(x.shape[0], -1)
        bound = D * 2.0 ** -24 * (x @ np.abs(to_np(p[w]).astype(np.float64)).T)
        allowed = _bf16_spacing(np.maximum(np.abs(g), np.abs(ref_k))) + bound
        diff = np.abs(g - ref_k)
        frac = float(np.mean(diff > 0))
        print(f"  {what} {key}: max diff / allowed {float((diff / allowed).max()):.3f}, "
              f"{frac:.2e} of elements differ", flush=True)
        assert np.all(diff <= allowed) and frac < 1e-3, (what, key)
    for key in ("alpha", "beta"):
        err = float(np.abs(to_np(r[key]).astype(np.float64) - ref[key]).max())
        assert err < 1e-6, (what, key, err)


@pytest.mark.parametrize("gen_bias", [False, True])
@pytest.mark.parametrize("B,T,H,dk,dv,D", [(2, 70, 3, 64, 128, 256), (1, 33, 2, 32, 64, 128), (1, 300, 12, 96, 256, 1536)])
def test_project_vs_oracle(jb, oracle_mod, gen_bias, B, T, H, dk, dv, D):
    """q, k, v, the gates (with their biases) and the generator taps (with and without the
    generator's biases) from one jb_project call."""
    from gated_delta_rule_jetblock_amd import inputs
    print(f"project B={B} T={T} H={H} dk={dk} dv={dv} D={D} gen_bias={gen_bias}", flush=True)
    s = inputs.Shape(B=B, T=T, H=H, dk=dk, dv=dv, d_model=D)
    p = inputs.projection_inputs(s, seed=T + D)
    if gen_bias:
        g = torch.Generator().manual_seed(T)
        p["b1"] = (torch.randn(32, generator=g) * 0.3).to(torch.bfloat16)
        p["b2"] = (torch.randn(4 * H, generator=g) * 0.3).to(torch.bfloat16)
    d = {k: v.cuda() for k, v in p.items()}
    r = jb.project(**d)
    torch.cuda.synchronize()
    a = _oracle_args(p)
    ref = oracle_mod.project(a["x"], a["Wq"], a["Wk"], a["Wv"], a["Wa"], a["Wb"], ba=a["ba"], bb=a["bb"])
    _check_projections(r, ref, p, f"T={T}")
    taps = oracle_mod.gen_taps(a["x"], a["W1"], a["W2"], b1=to_np(p.get("b1")), b2=to_np(p.get("b2")), H=H)
    assert rel_err(r["taps"], taps) < 1e-5


@pytest.mark.parametrize("B,T,H,dk,dv,D", [(1, 4133, 3, 64, 128, 256), (1, 4133, 16, 128, 256, 2048)])
def test_project_large_tiles_vs_oracle(jb, oracle_mod, B, T, H, dk, dv, D):
    """The 256 x 256 tile configuration (4096 tokens and more): a token tail of 37 rows, feature
    tiles that straddle q / k / v (H dk = 192), and the 4B widths (d_model 2048, 8192 q/k/v
    features); the generator tile with its biases."""
    from gated_delta_rule_jetblock_amd import inputs
    print(f"project (large tiles) B={B} T={T} H={H} dk={dk} dv={dv} D={D}", flush=True)
    s = inputs.Shape(B=B, T=T, H=H, dk=dk, dv=dv, d_model=D)
    p = inputs.projection_inputs(s, seed=T + D + H)
    g = torch.Generator().manual_seed(H)
    p["b1"] = (torch.randn(32, generator=g) * 0.3).to(torch.bfloat16)
    p["b2"] = (torch.randn(4 * H, generator=g) * 0.3).to(torch.bfloat16)
    d = {k: v.cuda() for k, v in p.items()}
    r = jb.project(**d)
    torch.cuda.synchronize()
    a = _oracle_args(p)
    ref = oracle_mod.project(a["x"], a["Wq"], a["Wk"], a["Wv"], a["Wa"], a["Wb"], ba=a["ba"], bb=a["bb"])
    _check_projections(r, ref, p, f"T={T}")
    taps = oracle_mod.gen_taps(a["x"], a["W1"], a["W2"], b1=to_np(p["b1"]), b2=to_np(p["b2"]), H=H)
    assert rel_err(r["taps"], taps) < 1e-5


@pytest.mark.parametrize("B,T,H,dk,dv,D,seg", [(2, 70, 3, 64, 128, 256, None), (1, 200, 2, 96, 256, 512, 1),
                                               (1, 4096, 12, 96, 256, 1536, None)])
def test_prefill_from_x_vs_oracle(jb, oracle_mod, B, T, H, dk, dv, D, seg):
    """The whole block from x: projections, generator and the chunked recurrence (bench
    launch configuration at the 2B shape, T = 4096), against the oracle's projection + block."""
    from gated_delta_rule_jetblock_amd import inputs
    print(f"prefill_from_x B={B} T={T} H={H} dk={dk} dv={dv} D={D} seg={seg}", flush=True)
    s = inputs.Shape(B=B, T=T, H=H, dk=dk, dv=dv, d_model=D)
    p = inputs.projection_inputs(s, seed=5 + T)
    st = inputs.state_inputs(s, seed=5 + T)
    d = {k: v.cuda() for k, v in p.items()}
    r = jb.prefill_from_x(**d, S0=st["S"].cuda(), conv_in=st["cache"].cuda(), seg_len=seg)
    torch.cuda.synchronize()
    a = _oracle_args(p)
    ref = oracle_mod.prefill_from_x(a["x"], a["Wq"], a["Wk"], a["Wv"], a["Wa"], a["Wb"], a["W1"], a["W2"],
                                    ba=a["ba"], bb=a["bb"], S0=to_np(st["S"]), conv_in=to_np(st["cache"]))
    eo, es = rel_err(r["o"], ref["o"]), rel_err(r["S_final"], ref["S_final"])
    print(f"  o_err={eo:.3e} S_err={es:.3e}", flush=True)
    assert eo < TOL_BF16 and es < TOL_BF16
    # the conv cache out holds the last three projected value rows
    assert rel_err(r["conv_out"], ref["conv_out"]) < 2.0 ** -7


def test_prefill_from_x_empty_sequence_passes_state(jb):
    from gated_delta_rule_jetblock_amd import inputs
    s = inputs.Shape(B=2, T=0, H=2, dk=32, dv=64, d_model=128)
    p = {k: v.cuda() for k, v in inputs.projection_inputs(s).items()}
    st = inputs.state_inputs(s)
    S0, cache = st["S"].cuda(), st["cache"].cuda()
    r = jb.prefill_from_x(**p, S0=S0, conv_in=cache)
    torch.cuda.synchronize()
    assert torch.equal(r["S_final"], S0) and torch.equal(r["conv_out"], cache)


@pytest.mark.parametrize("B,H,dk,dv,D", [(256, 12, 96, 256, 1536), (5, 3, 64, 128, 256)])
def test_decode_step_from_x_vs_oracle(jb, oracle_mod, B, H, dk, dv, D):
    """Three decode steps from x_t (2B decode shape and a small one) against the oracle's
    projections + block step, on sampled sequences; and against jb_project followed by
    jb_decode_step (the step from x forms its gates inside the decode kernel, in another
    summation order than the projection GEMM, so the two agree to fp32 rounding)."""
    from gated_delta_rule_jetblock_amd import inputs
    print(f"decode_step_from_x B={B} H={H} dk={dk} dv={dv} D={D}", flush=True)
    s = inputs.Shape(B=B, T=3, H=H, dk=dk, dv=dv, d_model=D)
    p = inputs.projection_inputs(s, seed=B + D)          # x [B, 3, D]: three steps of x_t
    st = inputs.state_inputs(s, seed=B)
    d = {k: v.cuda() for k, v in p.items()}
    W = {k: d[k] for k in ("Wq", "Wk", "Wv", "Wa", "Wb", "W1", "W2", "ba", "bb")}
    S, cache = st["S"].cuda().clone(), st["cache"].cuda().clone()
    S2, cache2 = S.clone(), cache.clone()
    outs = []
    for t in range(3):
        xt = d["x"][:, t].contiguous()
        r = jb.decode_step_from_x(S, cache, xt, **W)
        outs.append(r["o"].clone())
        pr = jb.project(xt.view(B, 1, D), **W)
        r2 = jb.decode_step(S2, cache2, xt, pr["q"].view(B, H, dk), pr["k"].view(B, H, dk), pr["v"].view(B, H, dv),
                            pr["alpha"].view(B, H), pr["beta"].view(B, H), W["W1"], W["W2"])
        assert rel_err(r["o"], to_np(r2["o"])) < 1e-5
    torch.cuda.synchronize()
    assert rel_err(S, to_np(S2)) < 1e-5 and torch.equal(cache, cache2)
    bs = np.array(sorted({0, B // 2, B - 1}))
    a = _oracle_args(p)
    So, co = to_np(st["S"])[bs], to_np(st["cache"])[bs]
    worst = 0.0
    for t in range(3):
        xt = a["x"][bs, t:t + 1]
        pr = oracle_mod.project(xt, a["Wq"], a["Wk"], a["Wv"], a["Wa"], a["Wb"], ba=a["ba"], bb=a["bb"])
        ro = oracle_mod.decode_step(So, co, xt[:, 0], pr["q"][:, 0], pr["k"][:, 0], pr["v"][:, 0],
                                    pr["alpha"][:, 0].astype(np.float32), pr["beta"][:, 0].astype(np.float32),
                                    a["W1"], a["W2"])
        worst = max(worst, rel_err(outs[t][bs], ro["o"]))
        So, co = ro["S"], ro["cache"]
    es = rel_err(S[bs], So)
    print(f"  o_err={worst:.3e} S_err={es:.3e}", flush=True)
    assert worst < TOL_BF16 and es < TOL_BF16
