"""GPU parity of the static-conv Gated DeltaNet block (jb_prefill_static,
jb_decode_step_static) against the fp64 oracle (jbo_prefill_static): outputs and final
states within the bf16-input bar (1e-5 in the all-fp32 decode), the cache tails bit-exact
(they are copies of raw rows)."""
import numpy as np
import pytest
import torch

from helpers import TOL_BF16, TOL_F32, rel_err, to_np

pytestmark = pytest.mark.gpu

from gated_delta_rule_jetblock_amd.inputs import Shape, prefill_inputs, state_inputs, static_conv_inputs


@pytest.fixture(scope="module")
def jb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_jetblock_amd import jetblock
    return jetblock


def _inputs(shape, seed, with_cache=True, with_state=True):
    p = prefill_inputs(shape, seed=seed)
    w = static_conv_inputs(shape, seed=seed)
    d = {k: p[k] for k in ("q", "k", "v", "alpha", "beta")}
    d.update(wq=w["wq"], wk=w["wk"], wv=w["wv"])
    if with_cache:
        d.update(cache_q=w["cache_q"], cache_k=w["cache_k"], cache_v=w["cache_v"])
    if with_state:
        d["S0"] = state_inputs(shape, seed=seed)["S"]
    return d


def _heads(d, heads, dk, dv):
    """The inputs restricted to a subset of heads (weights by row blocks)."""
    out = {}
    for key, t in d.items():
        a = to_np(t)
        if key in ("wq", "wk"):
            a = np.concatenate([a[h * dk:(h + 1) * dk] for h in heads])
        elif key == "wv":
            a = np.concatenate([a[h * dv:(h + 1) * dv] for h in heads])
        elif key == "S0":
            a = a[:, heads]
        elif key.startswith("cache"):
            a = a[:, :, heads]
        else:
            a = a[:, :, heads]
        out[key] = np.ascontiguousarray(a)
    return out


def _run_gpu(jb, d, out_dtype=torch.float32, seg_len=None):
    g = {k: v.cuda() for k, v in d.items()}
    r = jb.prefill_static(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["wq"], g["wk"], g["wv"],
                          S0=g.get("S0"), cache_q=g.get("cache_q"), cache_k=g.get("cache_k"),
                          cache_v=g.get("cache_v"), out_dtype=out_dtype, seg_len=seg_len)
    torch.cuda.synchronize()
    return r


def _oracle(oracle_mod, d, heads=None, dk=None, dv=None, nthreads=None):
    a = _heads(d, heads, dk, dv) if heads is not None else {k: to_np(v) for k, v in d.items()}
    return oracle_mod.prefill_static(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["wq"], a["wk"], a["wv"],
                                     S0=a.get("S0"), cache_q=a.get("cache_q"), cache_k=a.get("cache_k"),
                                     cache_v=a.get("cache_v"), nthreads=nthreads)


# a bf16 output adds one rounding: at most 2^-9 of the element, so of the largest one
BF16_OUT = 2.0 ** -9


def _o_tol(tol, o):
    return tol + (BF16_OUT if o.dtype == torch.bfloat16 else 0.0)


def _check(r, ref, tol, what):
    e_o = rel_err(r["o"], ref["o"])
    e_s = rel_err(r["S_final"], ref["S_final"])
    print(f"  {what}: o {e_o:.2e}  S_final {e_s:.2e}", flush=True)
    assert e_o < _o_tol(tol, r["o"]) and e_s < tol, (what, e_o, e_s)
    for key in ("cache_q", "cache_k", "cache_v"):
        if r.get(key) is not None:
            assert np.array_equal(to_np(r[key]), ref[key]), (what, key)


@pytest.mark.parametrize("B,T,H,dk,dv,seg_len,cache,state,out", [
    (2, 200, 2, 32, 64, None, True, True, "f32"),      # 3 chunks + a ragged tail, caches and S0
    (2, 200, 2, 32, 64, None, False, False, "bf16"),   # zero caches and state, bf16 o
    (1, 300, 3, 64, 128, 2, True, True, "f32"),        # several segments (summary + scan)
    (1, 1000, 2, 96, 256, 4, True, True, "f32"),
    (1, 130, 1, 128, 256, None, True, True, "f32"),
    (2, 2, 2, 32, 64, None, True, True, "f32"),        # shorter than the conv: the caches feed every row
    (3, 1, 1, 64, 128, None, True, False, "f32"),
])
def test_prefill_static_vs_oracle(jb, oracle_mod, B, T, H, dk, dv, seg_len, cache, state, out):
    print(f"[prefill_static B={B} T={T} H={H} dk={dk} dv={dv} seg={seg_len} cache={cache} state={state} o={out}]",
          flush=True)
    shape = Shape(B=B, T=T, H=H, dk=dk, dv=dv, d_model=128)
    d = _inputs(shape, seed=B * 1000 + T, with_cache=cache, with_state=state)
    r = _run_gpu(jb, d, torch.float32 if out == "f32" else torch.bfloat16, seg_len)
    ref = _oracle(oracle_mod, d)
    _check(r, ref, TOL_BF16, "prefill_static")


def test_prefill_static_empty_sequence(jb, oracle_mod):
    """T = 0: the state passes through and each cache is copied unchanged."""
    shape = Shape(B=2, T=0, H=2, dk=32, dv=64, d_model=128)
    d = _inputs(shape, seed=3)
    r = _run_gpu(jb, d)
    assert torch.equal(r["S_final"].cpu(), d["S0"])
    for key in ("cache_q", "cache_k", "cache_v"):
        assert torch.equal(r[key].cpu(), d[key]), key


def test_prefill_static_jetblock2b_T4096(jb, oracle_mod):
    """The 2B head shape (H = 12, dk = 96, dv = 256) at T = 4096, every head."""
    shape = Shape(B=1, T=4096, H=12, dk=96, dv=256, d_model=1536)
    print("[prefill_static 2B T=4096]", flush=True)
    d = _inputs(shape, seed=11)
    r = _run_gpu(jb, d)
    ref = _oracle(oracle_mod, d)
    _check(r, ref, TOL_BF16, "2B T=4096")


def test_prefill_static_jetblock2b_T65536_sampled_heads(jb, oracle_mod):
    """The full 64K-token 2B workload in the segment split the library picks, checked on two
    heads the oracle recomputes from scratch (the first and the last)."""
    shape = Shape(B=1, T=65536, H=12, dk=96, dv=256, d_model=1536)
    print("[prefill_static 2B T=65536, heads 0 and 11]", flush=True)
    d = _inputs(shape, seed=12)
    r = _run_gpu(jb, d)
    heads = [0, 11]
    ref = _oracle(oracle_mod, d, heads=heads, dk=96, dv=256, nthreads=2)
    sub = dict(o=r["o"][:, :, heads], S_final=r["S_final"][:, heads])
    for key in ("cache_q", "cache_k", "cache_v"):
        sub[key] = r[key][:, :, heads]
    _check(sub, ref, TOL_BF16, "2B T=65536 heads 0, 11")


@pytest.mark.parametrize("B,H,dk,dv,io,out", [
    (4, 2, 32, 64, "bf16", "f32"),
    (4, 2, 32, 64, "f32", "f32"),
    (3, 3, 128, 128, "bf16", "bf16"),
    (256, 12, 96, 256, "bf16", "f32"),
])
def test_decode_step_static_vs_oracle(jb, oracle_mod, B, H, dk, dv, io, out):
    """Four decode steps in a row, in place on the state and the caches, each against the
    oracle's step from the oracle's previous state."""
    print(f"[decode_step_static B={B} H={H} dk={dk} dv={dv} io={io} o={out}]", flush=True)
    shape = Shape(B=B, T=4, H=H, dk=dk, dv=dv, d_model=128, io_dtype=io)
    d = _inputs(shape, seed=B + H)
    tol = TOL_F32 if io == "f32" else TOL_BF16
    S = d["S0"].cuda().clone()
    caches = {k: d[k].cuda().clone() for k in ("cache_q", "cache_k", "cache_v")}
    w = {k: d[k].cuda() for k in ("wq", "wk", "wv")}
    ref_S = to_np(d["S0"])
    ref_c = {k: to_np(d[k]) for k in caches}
    for t in range(4):
        xt = {k: d[k][:, t].contiguous() for k in ("q", "k", "v", "alpha", "beta")}
        g = {k: v.cuda() for k, v in xt.items()}
        r = jb.decode_step_static(S, caches["cache_q"], caches["cache_k"], caches["cache_v"], g["q"], g["k"], g["v"],
                                  g["alpha"], g["beta"], w["wq"], w["wk"], w["wv"],
                                  out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
        torch.cuda.synchronize()
        ref = oracle_mod.decode_step_static(ref_S, ref_c["cache_q"], ref_c["cache_k"], ref_c["cache_v"],
                                            to_np(xt["q"]), to_np(xt["k"]), to_np(xt["v"]), to_np(xt["alpha"]),
                                            to_np(xt["beta"]), to_np(d["wq"]), to_np(d["wk"]), to_np(d["wv"]))
        e_o, e_s = rel_err(r["o"], ref["o"]), rel_err(S, ref["S"])
        print(f"  step {t}: o {e_o:.2e}  S {e_s:.2e}", flush=True)
        assert e_o < _o_tol(tol, r["o"]) and e_s < tol, (t, e_o, e_s)
        for k in caches:
            assert np.array_equal(to_np(caches[k]), ref[k]), (t, k)
        ref_S = ref["S"]
        ref_c = {k: ref[k] for k in caches}


def test_prefill_then_decode_static_continues_the_sequence(jb, oracle_mod):
    """Prefill of T tokens, then one decode step from its state and caches, equals the
    oracle's prefill of T + 1 tokens (last output, final state and caches)."""
    shape = Shape(B=2, T=101, H=2, dk=64, dv=128, d_model=128)
    d = _inputs(shape, seed=21)
    head = {k: (v[:, :100].contiguous() if k in ("q", "k", "v", "alpha", "beta") else v) for k, v in d.items()}
    r = _run_gpu(jb, head)
    xt = {k: d[k][:, 100].contiguous().cuda() for k in ("q", "k", "v", "alpha", "beta")}
    w = {k: d[k].cuda() for k in ("wq", "wk", "wv")}
    S = r["S_final"]
    rd = jb.decode_step_static(S, r["cache_q"], r["cache_k"], r["cache_v"], xt["q"], xt["k"], xt["v"], xt["alpha"],
                               xt["beta"], w["wq"], w["wk"], w["wv"])
    torch.cuda.synchronize()
    ref = _oracle(oracle_mod, d)
    e_o = rel_err(rd["o"], ref["o"][:, 100])
    e_s = rel_err(S, ref["S_final"])
    print(f"  continuation: o {e_o:.2e}  S {e_s:.2e}", flush=True)
    assert e_o < TOL_BF16 and e_s < TOL_BF16
    for key in ("cache_q", "cache_k", "cache_v"):
        assert np.array_equal(to_np(rd[key]), ref[key]), key
