"""jb_prefill_noalloc, the prefill for callers that cannot allocate, against jb_prefill:
two calls in a row through the C ABI, the second on a smaller input, each identical bit
for bit to jb_prefill on the same inputs (the same kernels and segment plan on a
different workspace), and a shape whose workspace exceeds the array rejected on the
host before anything is launched."""
import ctypes

import pytest
import torch

from helpers import to_dev

from gated_delta_rule_jetblock_amd.inputs import Shape, prefill_inputs, state_inputs

# a 2B-shape head set at T = 4096 (segment maps and taps, 43.5 MiB of the 64), then
# a small ragged case with an initial state and conv cache
CASES = [
    (Shape(B=1, T=4096, H=12, dk=96, dv=256, d_model=1536), False, None),
    (Shape(B=2, T=300, H=2, dk=32, dv=64, d_model=128), True, 2),
]


@pytest.fixture(scope="module")
def jb():
    from gated_delta_rule_jetblock_amd import jetblock
    return jetblock


def _args(jb, s, seed, with_state):
    d = to_dev(prefill_inputs(s, seed=seed))
    st = state_inputs(s, seed=seed)
    extra = dict(S0=st["S"].cuda(), conv_in=st["cache"].cuda()) if with_state else {}
    return (d["x"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["W1"], d["W2"]), extra


@pytest.mark.gpu
def test_noalloc_matches_prefill_two_calls(jb):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for i, (s, with_state, seg) in enumerate(CASES):
        print(f"[noalloc call {i}: B={s.B} T={s.T} H={s.H} dk={s.dk} dv={s.dv} state={with_state}]", flush=True)
        need = jb.prefill_workspace_size(jb.make_shape(s.B, s.T, s.H, s.dk, s.dv, s.d_model, jb.JB_BF16,
                                                       jb.JB_BF16, jb.flag_segment(seg) if seg else 0))
        assert need <= jb.NOALLOC_SCRATCH_BYTES, need
        args, extra = _args(jb, s, 40 + i, with_state)
        kw = dict(out_dtype=torch.bfloat16, seg_len=seg, **extra)
        ref = jb.prefill(*args, **kw)
        got = jb.prefill_noalloc(*args, **kw)
        torch.cuda.synchronize()
        for name in ("o", "S_final", "conv_out"):
            assert torch.isfinite(ref[name].float()).all(), name
            assert torch.equal(got[name], ref[name]), (i, name)
        # the array keeps the last call's contents; a repeat on it changes nothing
        again = jb.prefill_noalloc(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(again["o"], ref["o"]) and torch.equal(again["S_final"], ref["S_final"])


def test_noalloc_rejects_shapes_above_the_array(jb):
    """B = 1, T = 65536, H = 12 needs 68 MiB: JB_ERR_WORKSPACE from the host check.  The
    pointers are aligned stand-ins that the library never dereferences: every check runs
    on the host before the first HIP call, the pointers' first (a NULL x is named)."""
    s = jb.make_shape(1, 65536, 12, 96, 256, 1536, jb.JB_BF16, jb.JB_BF16)
    assert jb.prefill_workspace_size(s) > jb.NOALLOC_SCRATCH_BYTES
    stand_in = ctypes.c_void_p(1 << 20)
    st = jb.library().jb_prefill_noalloc(ctypes.byref(s), *([stand_in] * 15), None)
    assert st == jb.JB_ERR_WORKSPACE, (st, jb.last_error())
    assert "jb_prefill_noalloc" in jb.last_error() and "workspace" in jb.last_error()
    st = jb.library().jb_prefill_noalloc(ctypes.byref(s), None, *([stand_in] * 14), None)
    assert st == jb.JB_ERR_INVALID_ARG and "x is NULL" in jb.last_error(), (st, jb.last_error())
