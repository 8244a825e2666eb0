"""GPU parity of packed batches of sequences of different lengths (jb_prefill_varlen)
against the fp64 oracle run on each sequence alone, the hand-off of their states and
caches to jb_decode_step, and bitwise agreement with jb_prefill when every length is equal."""
import numpy as np
import pytest
import torch

from helpers import TOL_BF16, rel_err, to_np

pytestmark = pytest.mark.gpu

from gated_delta_rule_jetblock_amd.inputs import Shape, packed_prefill_inputs, request_lengths, state_inputs


@pytest.fixture(scope="module")
def jb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_jetblock_amd import jetblock
    return jetblock


def _states(B, H, dk, dv, seed):
    st = state_inputs(Shape(B=B, T=1, H=H, dk=dk, dv=dv, d_model=128), seed=seed)
    return st["S"], st["cache"]


def _oracle_seq(oracle_mod, p, n, S0, cache, heads=None):
    """The oracle on sequence n of the packed batch alone (optionally a subset of heads)."""
    cu = p["cu_seqlens"].tolist()
    a, b = cu[n], cu[n + 1]
    sl = slice(a, b)
    hs = slice(None) if heads is None else heads
    W2 = to_np(p["W2"])
    if heads is not None:
        W2 = W2[np.concatenate([np.arange(h * 4, h * 4 + 4) for h in heads])]
    return oracle_mod.prefill(to_np(p["x"][sl])[None], np.ascontiguousarray(to_np(p["q"][sl])[:, hs][None]),
                              np.ascontiguousarray(to_np(p["k"][sl])[:, hs][None]),
                              np.ascontiguousarray(to_np(p["v"][sl])[:, hs][None]),
                              np.ascontiguousarray(to_np(p["alpha"][sl])[:, hs][None]),
                              np.ascontiguousarray(to_np(p["beta"][sl])[:, hs][None]), to_np(p["W1"]),
                              np.ascontiguousarray(W2),
                              S0=None if S0 is None else np.ascontiguousarray(to_np(S0[n:n + 1])[:, hs]),
                              conv_in=None if cache is None else np.ascontiguousarray(to_np(cache[n:n + 1])[:, :, hs]))


def _run(jb, p, S0=None, cache=None, seg_len=None, out_dtype=torch.float32):
    g = {k: v.cuda() for k, v in p.items()}
    r = jb.prefill_varlen(g["cu_seqlens"], g["x"], g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["W1"], g["W2"],
                          S0=None if S0 is None else S0.cuda(), conv_in=None if cache is None else cache.cuda(),
                          seg_len=seg_len, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("lengths,seg_len,state", [
    ([200, 0, 1, 2, 63, 64, 65, 130], None, True),   # empty, shorter than the conv, chunk edges
    ([1000, 37, 513, 0, 256], 2, True),               # several segments for the long ones only
    ([300, 300, 300], None, False),                    # zero initial state and cache
])
def test_varlen_vs_oracle_per_sequence(jb, oracle_mod, lengths, seg_len, state):
    H, dk, dv, D = 2, 64, 128, 128
    print(f"[varlen lengths={lengths} seg={seg_len} state={state}]", flush=True)
    p = packed_prefill_inputs(lengths, H, dk, dv, D, seed=len(lengths))
    S0, cache = _states(len(lengths), H, dk, dv, seed=5) if state else (None, None)
    r = _run(jb, p, S0, cache, seg_len)
    cu = p["cu_seqlens"].tolist()
    for n in range(len(lengths)):
        ref = _oracle_seq(oracle_mod, p, n, S0, cache)
        if lengths[n] > 0:
            e_o = rel_err(r["o"][cu[n]:cu[n + 1]], ref["o"][0])
        else:
            e_o = 0.0
        e_s = rel_err(r["S_final"][n], ref["S_final"][0])
        print(f"  seq {n} (T={lengths[n]}): o {e_o:.2e}  S {e_s:.2e}", flush=True)
        assert e_o < TOL_BF16 and e_s < TOL_BF16, (n, e_o, e_s)
        assert np.array_equal(to_np(r["conv_out"][n]), ref["conv_out"][0]), n


def test_varlen_equal_lengths_match_dense_bitwise(jb):
    """Four sequences of 700 tokens packed: the same plan and arithmetic as jb_prefill on
    [4, 700], so every output is bit-identical."""
    H, dk, dv, D = 3, 96, 256, 256
    p = packed_prefill_inputs([700] * 4, H, dk, dv, D, seed=9)
    S0, cache = _states(4, H, dk, dv, seed=9)
    r = _run(jb, p, S0, cache)
    g = {k: v.cuda() for k, v in p.items()}
    rd = jb.prefill(g["x"].view(4, 700, D), g["q"].view(4, 700, H, dk), g["k"].view(4, 700, H, dk),
                    g["v"].view(4, 700, H, dv), g["alpha"].view(4, 700, H), g["beta"].view(4, 700, H), g["W1"],
                    g["W2"], S0=S0.cuda(), conv_in=cache.cuda())
    torch.cuda.synchronize()
    assert torch.equal(r["o"].view(4, 700, H, dv), rd["o"])
    assert torch.equal(r["S_final"], rd["S_final"])
    assert torch.equal(r["conv_out"], rd["conv_out"])


def test_varlen_hands_off_to_decode(jb, oracle_mod):
    """Prefill a packed batch, then one jb_decode_step for all its sequences from the
    prefill's S_final and conv_out: each sequence's decode output equals the oracle's
    prefill of that sequence extended by the decoded token."""
    H, dk, dv, D = 2, 64, 128, 128
    lengths = [150, 3, 64, 99]
    full = [t + 1 for t in lengths]
    pf = packed_prefill_inputs(full, H, dk, dv, D, seed=13)
    cu_f = pf["cu_seqlens"].tolist()
    keep = torch.cat([torch.arange(cu_f[n], cu_f[n + 1] - 1) for n in range(len(lengths))])
    last = torch.tensor([cu_f[n + 1] - 1 for n in range(len(lengths))])
    p = {k: (v[keep] if k not in ("W1", "W2", "cu_seqlens") else v) for k, v in pf.items()}
    cu = [0]
    for t in lengths:
        cu.append(cu[-1] + t)
    p["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32)
    S0, cache = _states(len(lengths), H, dk, dv, seed=13)
    r = _run(jb, p, S0, cache)
    S, cc = r["S_final"], r["conv_out"]
    t = {k: pf[k][last].contiguous().cuda() for k in ("x", "q", "k", "v", "alpha", "beta")}
    rd = jb.decode_step(S, cc, t["x"], t["q"], t["k"], t["v"], t["alpha"], t["beta"], pf["W1"].cuda(),
                        pf["W2"].cuda())
    torch.cuda.synchronize()
    for n in range(len(lengths)):
        ref = _oracle_seq(oracle_mod, pf, n, S0, cache)
        e_o = rel_err(rd["o"][n], ref["o"][0, -1])
        e_s = rel_err(S[n], ref["S_final"][0])
        print(f"  seq {n}: decode o {e_o:.2e}  S {e_s:.2e}", flush=True)
        assert e_o < TOL_BF16 and e_s < TOL_BF16, (n, e_o, e_s)
        assert np.array_equal(to_np(cc[n]), ref["conv_out"][0]), n


def test_varlen_serving_batch_jetblock2b(jb, oracle_mod):
    """A serving batch at the 2B head shape: 32 requests of 2K..8K tokens (the short-context
    regime), checked on three sequences (shortest, longest, one more) and two heads each."""
    H, dk, dv, D = 12, 96, 256, 1536
    lengths = request_lengths(32, 2048, 8192, seed=1)
    print(f"[varlen 2B serving batch: {len(lengths)} requests, {sum(lengths)} tokens]", flush=True)
    p = packed_prefill_inputs(lengths, H, dk, dv, D, seed=17)
    S0, cache = _states(len(lengths), H, dk, dv, seed=17)
    r = _run(jb, p, S0, cache, out_dtype=torch.bfloat16)
    cu = p["cu_seqlens"].tolist()
    picks = sorted({int(np.argmin(lengths)), int(np.argmax(lengths)), 7})
    heads = [0, 11]
    for n in picks:
        ref = _oracle_seq(oracle_mod, p, n, S0, cache, heads=heads)
        e_o = rel_err(r["o"][cu[n]:cu[n + 1]][:, heads].float(), ref["o"][0])
        e_s = rel_err(r["S_final"][n][heads], ref["S_final"][0])
        print(f"  seq {n} (T={lengths[n]}): o {e_o:.2e}  S {e_s:.2e}", flush=True)
        # bf16 o: one more rounding, at most 2^-9 of the largest element
        assert e_o < TOL_BF16 + 2.0 ** -9 and e_s < TOL_BF16, (n, e_o, e_s)


def test_malformed_offsets_stay_in_bounds(jb):
    """cu_seqlens lives in device memory, so the host cannot validate it: offsets past the
    packed rows, negative and decreasing offsets give wrong rows but no access outside the
    tensors.  o, S_final and conv_out sit inside NaN-filled buffers whose guard regions on
    both sides must keep their fill."""
    print("[malformed cu_seqlens]", flush=True)
    H, dk, dv, D, total, Tmax = 2, 32, 64, 128, 300, 200
    p = packed_prefill_inputs([100, 100, 100], H, dk, dv, D, seed=3)
    g = {k: v.cuda() for k, v in p.items()}
    bad = torch.tensor([0, 500, -40, 300], dtype=torch.int32, device="cuda")
    guard = 4096

    def guarded(n, dtype):
        buf = torch.full((guard + n + guard,), float("nan"), dtype=dtype, device="cuda")
        return buf, buf[guard:guard + n]

    ob, o = guarded(total * H * dv, torch.float32)
    sb, s = guarded(3 * H * dk * dv, torch.float32)
    cb, c = guarded(3 * 3 * H * dv, torch.bfloat16)
    jb.prefill_varlen(bad, g["x"], g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["W1"], g["W2"],
                      max_seqlen=Tmax, o=o.view(total, H, dv), S_final=s.view(3, H, dk, dv),
                      conv_out=c.view(3, 3, H, dv), seg_len=1)
    torch.cuda.synchronize()
    for buf in (ob, sb, cb):
        assert torch.isnan(buf[:guard].float()).all() and torch.isnan(buf[-guard:].float()).all()
