"""The JetBlock 4B-shape workload as one chain, as the pages' long-context setting runs
it (Jet-Nemotron csdn translation, section 3.1: prefill of a long prompt, then decoding
from the state it leaves).  The GPU prefills B=1, T=262144, H=16, dk=128, dv=256,
d_model=2048 in the default segment plan, the final state and conv cache are copied to
a batch of 128 sequences, and jb_decode_step runs that batch for 128 steps with the
layer's own generator weights.  The oracle runs the same chain in fp64: its prefill over
all sixteen heads (every output and final state checked), then decode from its own final
state for a sample of the sequences, checked at every step."""
import numpy as np
import pytest
import torch

from helpers import TOL_BF16, oracle_prefill, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

DECODE_B = 128
STEPS = 128
SAMPLE = [0, 1, 31, 64, 100, 127]


@pytest.fixture(scope="module")
def jb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_jetblock_amd import jetblock
    return jetblock


def test_jetblock4b_prefill_then_decode(jb, oracle_mod):
    from gated_delta_rule_jetblock_amd import inputs
    s = inputs.B4_T262144
    print(f"[4B chain: prefill T={s.T} H={s.H}, then decode B={DECODE_B} x {STEPS}]", flush=True)
    p = inputs.prefill_inputs(s, seed=0)
    d = to_dev(p)
    r = jb.prefill(d["x"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["W1"], d["W2"])
    torch.cuda.synchronize()
    del d
    ref = oracle_prefill(oracle_mod, p)  # all sixteen heads
    eo = rel_err(r["o"], ref["o"])
    es = rel_err(r["S_final"], ref["S_final"])
    print(f"  prefill o_err={eo:.3e} S_err={es:.3e}", flush=True)
    assert eo < TOL_BF16 and es < TOL_BF16, (eo, es)
    np.testing.assert_array_equal(to_np(r["conv_out"]), ref["conv_out"])
    S_ref, cache_ref = ref["S_final"], ref["conv_out"]
    del ref
    r["o"] = None

    # the prefill's state and cache, one copy per sequence of the decode batch
    S = r["S_final"].expand(DECODE_B, -1, -1, -1).contiguous()
    cache = r["conv_out"].expand(DECODE_B, -1, -1, -1).contiguous()
    st = inputs.decode_inputs(inputs.B4_DECODE, steps=STEPS, seed=11, with_state=False)
    W1, W2 = p["W1"].cuda(), p["W2"].cuda()
    dev = {k: st[k].cuda() for k in ("x", "q", "k", "v", "alpha", "beta")}
    outs = []
    for t in range(STEPS):
        o = jb.decode_step(S, cache, dev["x"][t], dev["q"][t], dev["k"][t], dev["v"][t], dev["alpha"][t],
                           dev["beta"][t], W1, W2)["o"]
        outs.append(o[SAMPLE].clone())
    torch.cuda.synchronize()

    bs = np.array(SAMPLE)
    So = np.repeat(S_ref, len(bs), axis=0)
    co = np.repeat(cache_ref, len(bs), axis=0)
    W1n, W2n = to_np(p["W1"]), to_np(p["W2"])
    worst = 0.0
    for t in range(STEPS):
        ro = oracle_mod.decode_step(So, co, to_np(st["x"][t])[bs], to_np(st["q"][t])[bs], to_np(st["k"][t])[bs],
                                    to_np(st["v"][t])[bs], to_np(st["alpha"][t])[bs], to_np(st["beta"][t])[bs],
                                    W1n, W2n)
        e = rel_err(outs[t], ro["o"])
        assert e < TOL_BF16, (t, e)
        worst = max(worst, e)
        So, co = ro["S"], ro["cache"]
    eS = rel_err(S[SAMPLE], So)
    print(f"  decode worst o_err={worst:.3e} final S_err={eS:.3e}", flush=True)
    assert eS < TOL_BF16, eS
    np.testing.assert_array_equal(to_np(cache[SAMPLE]), co)
