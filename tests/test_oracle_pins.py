"""Pins of the fp64 oracle against facts fixed independently of its own code.

The block (Jet-Nemotron csdn translation, section 2.4; xugj520 blog, section 2.2):
kernel generator Linear -> SiLU -> Linear emitting conv taps, dynamic causal conv
of kernel size 4 on V only, Gated DeltaNet time mixing
S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v'_t k_t^T, o_t = S_t q_t over
L2-normalised q, k.  Each test below checks a property that a plausible slip
in the oracle (dropped term, wrong sign, wrong index, transposed operand,
off-by-one tap) would break.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _rand_block(B=1, T=7, H=2, dk=8, dv=5, D=16, G=4, K=4, seed=0, amean=1.0):
    r = np.random.default_rng(seed)
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    sig = lambda z: (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    return dict(x=f(B, T, D), q=f(B, T, H, dk), k=f(B, T, H, dk), v=f(B, T, H, dv),
                alpha=sig(f(B, T, H) + amean), beta=sig(f(B, T, H)),
                W1=f(G, D) * 0.3, W2=f(H * K, G) * 0.3)


def _unit(x, eps=1e-6):
    x = np.asarray(x, np.float64)
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def _hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


# ------------------------------------------------------------------ golden


def test_golden_hand_two_tokens(oracle_mod):
    """Hand-derived two-token example (tests/golden/hand_two_tokens.json)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_two_tokens.json")))
    inp = {k: np.array(v, np.float32) for k, v in g["inputs"].items()}
    for case in g["cases"]:
        r = oracle_mod.prefill(**inp, b2=np.array(case["b2"], np.float32))
        np.testing.assert_allclose(r["o"], np.array(case["o"]), atol=1e-12, err_msg=case["name"])
        np.testing.assert_allclose(r["S_final"], np.array(case["S_final"]), atol=1e-12,
                                   err_msg=case["name"])
        np.testing.assert_array_equal(r["conv_out"], np.array(case["conv_out"], np.float32))


# ------------------------------------------------------------ recurrence


def test_identity_gates_leave_state_unchanged(oracle_mod):
    """a = 1, b = 0: S_T = S_0 exactly, and o_t reads S_0 along q."""
    p = _rand_block(T=9, dk=8, dv=6)
    p["alpha"][:] = 1.0
    p["beta"][:] = 0.0
    S0 = RNG.standard_normal((1, 2, 8, 6)).astype(np.float32)
    # q = 1000 * e_i picks row i of M0 = S0^T (column i of S0)
    p["q"][:] = 0.0
    for t in range(9):
        p["q"][0, t, :, t % 8] = 1000.0
    r = oracle_mod.prefill(**p, S0=S0)
    np.testing.assert_array_equal(r["S_final"], S0.astype(np.float64))
    for t in range(9):
        np.testing.assert_allclose(r["o"][0, t], S0[0, :, t % 8, :], rtol=1e-12, atol=1e-12)


def test_pure_decay_when_beta_zero(oracle_mod):
    """b = 0: S_T = (prod a) S_0."""
    p = _rand_block(T=6)
    p["beta"][:] = 0.0
    S0 = RNG.standard_normal((1, 2, 8, 5)).astype(np.float32)
    r = oracle_mod.prefill(**p, S0=S0)
    decay = np.prod(p["alpha"][0].astype(np.float64), axis=0)  # [H]
    np.testing.assert_allclose(r["S_final"][0], decay[:, None, None] * S0[0], rtol=1e-13)


def test_orthonormal_keys_retrieve_written_values(oracle_mod):
    """a = 1, b = 1, orthonormal keys: S k_j = v'_j for every written pair, from any S_0,
    and a later write with the same key returns the newer value."""
    dk, dv, T = 16, 6, 10
    p = _rand_block(T=T, H=1, dk=dk, dv=dv)
    p["alpha"][:] = 1.0
    p["beta"][:] = 1.0
    # taps = b2 = (0,0,0,1): v'_t = v_t
    p["W1"][:] = 0.0
    p["W2"][:] = 0.0
    b2 = np.array([0, 0, 0, 1], np.float32)
    keys = _hadamard(dk)[:T] * 256.0  # exact in float32, norm 1024 -> eps invisible
    keys[T - 1] = keys[2]             # the last token re-writes key 2
    p["k"][0, :, 0, :] = keys
    p["q"][0, :, 0, :] = keys          # query = key: o_t reads the value just written
    S0 = RNG.standard_normal((1, 1, dk, dv)).astype(np.float32)
    r = oracle_mod.prefill(**p, b2=b2, S0=S0)
    v = p["v"][0, :, 0, :].astype(np.float64)
    np.testing.assert_allclose(r["o"][0, :, 0, :], v, rtol=0, atol=1e-11)
    M = r["S_final"][0, 0]
    khat = keys / np.linalg.norm(keys, axis=1, keepdims=True)
    for j in range(T - 1):
        want = v[T - 1] if j == 2 else v[j]
        np.testing.assert_allclose(M.T @ khat[j], want, atol=1e-11)


def test_single_token_from_zero(oracle_mod):
    """T = 1, S_0 = 0: S_1 = b v' k^T, o = b (k.q) v' (the updated state is read)."""
    p = _rand_block(T=1, H=1, dk=8, dv=5)
    p["W1"][:] = 0.0
    p["W2"][:] = 0.0
    b2 = np.array([0, 0, 0, 1], np.float32)
    r = oracle_mod.prefill(**p, b2=b2)
    kh = _unit(p["k"][0, 0, 0])
    qh = _unit(p["q"][0, 0, 0])
    v = p["v"][0, 0, 0].astype(np.float64)
    b = float(p["beta"][0, 0, 0])
    np.testing.assert_allclose(r["S_final"][0, 0], b * np.outer(kh, v), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(r["o"][0, 0, 0], b * (kh @ qh) * v, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("T", [1, 3, 8])
def test_closed_form_product_of_matrices(oracle_mod, T):
    """Explicit product form in the dv x dk orientation:
    S_T = S_0 A_1...A_T + sum_t b_t v'_t k_t^T A_{t+1}...A_T,  A_t = a_t (I - b_t k_t k_t^T),
    o_t = S_t q_t.  The oracle returns M = S^T."""
    H, dk, dv = 2, 6, 4
    p = _rand_block(T=T, H=H, dk=dk, dv=dv, seed=T)
    S0 = RNG.standard_normal((1, H, dk, dv)).astype(np.float32)
    r = oracle_mod.prefill(**p, S0=S0, want_taps=True)
    vc = oracle_mod.conv(r["taps"], p["v"])  # v' (pinned separately below)
    for h in range(H):
        kh = _unit(p["k"][0, :, h])
        qh = _unit(p["q"][0, :, h])
        a = p["alpha"][0, :, h].astype(np.float64)
        b = p["beta"][0, :, h].astype(np.float64)
        A = [a[t] * (np.eye(dk) - b[t] * np.outer(kh[t], kh[t])) for t in range(T)]

        def prod(lo, hi):  # A_lo ... A_{hi-1} (0-based, left to right)
            P = np.eye(dk)
            for t in range(lo, hi):
                P = P @ A[t]
            return P

        for tt in range(1, T + 1):
            S = S0[0, h].T.astype(np.float64) @ prod(0, tt)
            for t in range(tt):
                S = S + b[t] * np.outer(vc[0, t, h], kh[t]) @ prod(t + 1, tt)
            np.testing.assert_allclose(r["o"][0, tt - 1, h], S @ qh[tt - 1], rtol=1e-11,
                                       atol=1e-12)
        np.testing.assert_allclose(r["S_final"][0, h], S.T, rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------ conv


@pytest.mark.parametrize("j", [0, 1, 2, 3])
@pytest.mark.parametrize("with_cache", [False, True])
def test_one_hot_taps_shift(oracle_mod, j, with_cache):
    """Taps = e_j (W2 = 0, b2 one-hot): v'_t = v_{t-3+j}, zero-filled or read
    from the cache (oldest row first) before the start."""
    B, T, H, dv, K = 2, 7, 3, 5, 4
    p = _rand_block(B=B, T=T, H=H, dv=dv)
    p["W2"][:] = 0.0
    b2 = np.zeros(H * K, np.float32)
    b2[j::K] = 1.0
    cache = RNG.standard_normal((B, K - 1, H, dv)).astype(np.float32) if with_cache else None
    taps = oracle_mod.gen_taps(p["x"], p["W1"], p["W2"], b2=b2, H=H)
    vc = oracle_mod.conv(taps, p["v"], cache)
    hist = np.concatenate([cache if with_cache else np.zeros((B, K - 1, H, dv), np.float32),
                           p["v"]], axis=1)
    want = hist[:, j:j + T]  # index t - 3 + j in v  ==  t + j in hist
    np.testing.assert_array_equal(vc, want.astype(np.float64))


def test_conv_is_linear_in_v(oracle_mod):
    p = _rand_block(T=9)
    taps = oracle_mod.gen_taps(p["x"], p["W1"], p["W2"], H=2)
    # dyadic values so that v1 + 2 v2 is exact in the float32 inputs
    v1 = np.round(p["v"] * 16.0).astype(np.float32) / 16.0
    v2 = np.round(RNG.standard_normal(p["v"].shape) * 16.0).astype(np.float32) / 16.0
    a = oracle_mod.conv(taps, v1) + 2.0 * oracle_mod.conv(taps, v2)
    b = oracle_mod.conv(taps, v1 + 2.0 * v2)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_conv_out_holds_last_raw_rows(oracle_mod):
    for T in (1, 2, 3, 9):
        p = _rand_block(T=T, H=2, dv=5)
        cache = RNG.standard_normal((1, 3, 2, 5)).astype(np.float32)
        r = oracle_mod.prefill(**p, conv_in=cache)
        hist = np.concatenate([cache, p["v"]], axis=1)
        np.testing.assert_array_equal(r["conv_out"], hist[:, -3:])


# ------------------------------------------------------------- generator


def test_generator_silu_odd_part_and_zero():
    """SiLU(h) - SiLU(-h) = h and SiLU(0) = 0; SiLU(ln 3) = 0.75 ln 3."""
    import oracle
    D, G, H, K = 4, 3, 2, 4
    W2 = RNG.standard_normal((H * K, G)).astype(np.float32)
    b2 = RNG.standard_normal(H * K).astype(np.float32)
    x = np.zeros((3, D), np.float32)
    x[:, 1] = [1.0, -1.0, 0.0]
    W1 = np.zeros((G, D), np.float32)
    w = np.float32(np.log(3.0))
    W1[2, 1] = w
    t = oracle.gen_taps(x, W1, W2, b2=b2, H=H).reshape(3, H * K)
    col = W2[:, 2].astype(np.float64)
    np.testing.assert_allclose(t[2], b2.astype(np.float64), rtol=0, atol=0)  # SiLU(0) = 0
    np.testing.assert_allclose(t[0] - t[1], col * float(w), rtol=1e-12, atol=1e-14)
    # w is float32(ln 3), within 3e-8 of ln 3, so sigmoid(w) = 3/4 to 1e-8
    np.testing.assert_allclose(t[0] - b2, col * 0.75 * float(w), rtol=5e-8, atol=1e-14)


def test_generator_first_layer_bias_and_tap_layout():
    """Hidden unit g = SiLU(W1[g].x + b1[g]); tap j of head h is row h*K + j of W2."""
    import oracle
    D, G, H, K = 5, 4, 3, 4
    x = RNG.standard_normal((2, D)).astype(np.float32)
    W1 = np.zeros((G, D), np.float32)
    b1 = np.zeros(G, np.float32)
    b1[1] = np.float32(np.log(3.0))
    W2 = np.zeros((H * K, G), np.float32)
    W2[2 * K + 1, 1] = 1.0  # head 2, tap 1 reads hidden unit 1
    t = oracle.gen_taps(x, W1, W2, b1=b1, H=H)
    want = np.zeros((2, H, K))
    want[:, 2, 1] = 0.75 * float(np.float32(np.log(3.0)))
    np.testing.assert_allclose(t, want, rtol=5e-8, atol=1e-15)


# --------------------------------------------------------- normalisation


def test_l2norm_unit_and_scale_invariant():
    import oracle
    x = RNG.standard_normal((6, 96)).astype(np.float32)
    n = oracle.l2norm(x)
    np.testing.assert_allclose(np.linalg.norm(n, axis=1), 1.0, atol=1e-7)
    n4 = oracle.l2norm(4.0 * x)
    np.testing.assert_allclose(n4, n, atol=1e-8)
    # direction preserved: n is a positive multiple of x
    ratio = n / x.astype(np.float64)
    np.testing.assert_allclose(ratio, ratio[:, :1] * np.ones_like(ratio), rtol=1e-12)


def test_block_invariant_to_qk_scale(oracle_mod):
    p = _rand_block(T=6)
    r1 = oracle_mod.prefill(**p)
    p2 = dict(p, q=p["q"] * 8.0, k=p["k"] * 0.5)
    r2 = oracle_mod.prefill(**p2)
    np.testing.assert_allclose(r2["o"], r1["o"], rtol=1e-6, atol=1e-7)


# ------------------------------------------------------- whole block


def test_split_prefill_equals_full(oracle_mod):
    """Prefill [0,T1) then [T1,T) from (S_final, conv_out) equals one prefill."""
    p = _rand_block(B=2, T=11)
    S0 = RNG.standard_normal((2, 2, 8, 5)).astype(np.float32)
    full = oracle_mod.prefill(**p, S0=S0)
    T1 = 4
    a = {k: (v[:, :T1] if k in ("x", "q", "k", "v", "alpha", "beta") else v) for k, v in p.items()}
    b = {k: (v[:, T1:] if k in ("x", "q", "k", "v", "alpha", "beta") else v) for k, v in p.items()}
    ra = oracle_mod.prefill(**a, S0=S0)
    # the float32 hand-off of the state is the only rounding; compare loosely
    rb = oracle_mod.prefill(**b, S0=ra["S_final"].astype(np.float32), conv_in=ra["conv_out"])
    np.testing.assert_allclose(ra["o"], full["o"][:, :T1], rtol=0, atol=0)
    np.testing.assert_allclose(rb["o"], full["o"][:, T1:], rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(rb["S_final"], full["S_final"], rtol=1e-6, atol=1e-6)


def test_prefill_equals_decode_loop(oracle_mod):
    p = _rand_block(B=2, T=5)
    S0 = RNG.standard_normal((2, 2, 8, 5)).astype(np.float32)
    cache = RNG.standard_normal((2, 3, 2, 5)).astype(np.float32)
    full = oracle_mod.prefill(**p, S0=S0, conv_in=cache)
    S, c = S0, cache
    for t in range(5):
        d = oracle_mod.decode_step(S, c, p["x"][:, t], p["q"][:, t], p["k"][:, t], p["v"][:, t],
                                   p["alpha"][:, t], p["beta"][:, t], p["W1"], p["W2"])
        np.testing.assert_allclose(d["o"], full["o"][:, t], rtol=1e-6, atol=1e-6)
        S, c = d["S"].astype(np.float32), d["cache"]
    np.testing.assert_allclose(S, full["S_final"], rtol=1e-6, atol=1e-6)
    np.testing.assert_array_equal(c, full["conv_out"])


def test_sequences_and_heads_are_independent(oracle_mod):
    """Batch rows and heads do not mix: permuting heads permutes outputs."""
    p = _rand_block(B=2, T=6, H=3)
    r = oracle_mod.prefill(**p)
    perm = [2, 0, 1]
    K = 4
    p2 = dict(p)
    for key in ("q", "k", "v", "alpha", "beta"):
        p2[key] = np.ascontiguousarray(p[key][:, :, perm])
    rows = np.concatenate([np.arange(h * K, h * K + K) for h in perm])
    p2["W2"] = np.ascontiguousarray(p["W2"][rows])
    r2 = oracle_mod.prefill(**p2)
    np.testing.assert_allclose(r2["o"], r["o"][:, :, perm], rtol=1e-13, atol=1e-15)
    r1b = oracle_mod.prefill(**{k: (v[1:] if k in ("x", "q", "k", "v", "alpha", "beta") else v)
                                for k, v in p.items()})
    np.testing.assert_allclose(r1b["o"][0], r["o"][1], rtol=0, atol=0)


def test_threads_do_not_change_results(oracle_mod):
    p = _rand_block(B=3, T=8, H=3)
    r1 = oracle_mod.prefill(**p, nthreads=1)
    r4 = oracle_mod.prefill(**p, nthreads=4)
    np.testing.assert_array_equal(r1["o"], r4["o"])
    np.testing.assert_array_equal(r1["S_final"], r4["S_final"])
