"""CPU pins of the oracle's static-conv Gated DeltaNet block (jbo_prefill_static), the
block JetBlock replaces: reductions to the JetBlock oracle, shifted inputs, per-channel
weights against their definition, continuation through the caches, decode = prefill."""
import numpy as np
import pytest


@pytest.fixture(scope="module")
def oracle_mod():
    import oracle
    oracle.build()
    return oracle


def _inputs(B=2, T=11, H=2, dk=4, dv=6, seed=0):
    g = np.random.default_rng(seed)
    return dict(q=g.standard_normal((B, T, H, dk)).astype(np.float32),
                k=g.standard_normal((B, T, H, dk)).astype(np.float32),
                v=g.standard_normal((B, T, H, dv)).astype(np.float32),
                alpha=(1 / (1 + np.exp(-g.standard_normal((B, T, H)) - 2))).astype(np.float32),
                beta=(1 / (1 + np.exp(-g.standard_normal((B, T, H))))).astype(np.float32))


def _onehot(rows, j, K=4):
    w = np.zeros((rows, K), np.float32)
    w[:, j] = 1.0
    return w


def test_identity_weights_equal_jetblock_with_constant_taps(oracle_mod):
    """w = e_3 (the current token only) on q and k, and v weights equal per head: the static
    block is JetBlock with a generator whose output is that constant tap set (W1 = W2 = 0,
    b2 = taps).  Two code paths of the oracle must agree."""
    B, T, H, dk, dv = 2, 9, 2, 4, 6
    p = _inputs(B, T, H, dk, dv)
    g = np.random.default_rng(1)
    taps = g.standard_normal((H, 4)).astype(np.float32)
    wv = np.repeat(taps, dv, axis=0)                       # row h*dv + c = taps of head h
    cache_v = g.standard_normal((B, 3, H, dv)).astype(np.float32)
    S0 = g.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.1
    r = oracle_mod.prefill_static(**p, wq=_onehot(H * dk, 3), wk=_onehot(H * dk, 3), wv=wv, S0=S0, cache_v=cache_v)
    D = 8
    x = g.standard_normal((B, T, D)).astype(np.float32)
    ref = oracle_mod.prefill(x, **p, W1=np.zeros((32, D), np.float32), W2=np.zeros((4 * H, 32), np.float32),
                             b2=taps.reshape(-1), S0=S0, conv_in=cache_v)
    np.testing.assert_allclose(r["o"], ref["o"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["S_final"], ref["S_final"], rtol=1e-12, atol=1e-13)


def test_shift_weights_delay_the_inputs(oracle_mod):
    """w = e_0 on q, k and v: every token sees the inputs of three tokens earlier (the caches
    supply the first three), i.e. the identity-weight block on the delayed sequences."""
    B, T, H, dk, dv = 1, 10, 2, 4, 5
    p = _inputs(B, T, H, dk, dv, seed=4)
    g = np.random.default_rng(5)
    cq = g.standard_normal((B, 3, H, dk)).astype(np.float32)
    ck = g.standard_normal((B, 3, H, dk)).astype(np.float32)
    cv = g.standard_normal((B, 3, H, dv)).astype(np.float32)
    r = oracle_mod.prefill_static(**p, wq=_onehot(H * dk, 0), wk=_onehot(H * dk, 0), wv=_onehot(H * dv, 0),
                                  cache_q=cq, cache_k=ck, cache_v=cv)
    shift = lambda c, x: np.concatenate([c, x], axis=1)[:, :T]
    p2 = dict(p, q=shift(cq, p["q"]), k=shift(ck, p["k"]), v=shift(cv, p["v"]))
    ref = oracle_mod.prefill_static(**p2, wq=_onehot(H * dk, 3), wk=_onehot(H * dk, 3), wv=_onehot(H * dv, 3))
    np.testing.assert_allclose(r["o"], ref["o"], rtol=1e-13, atol=1e-14)


def test_per_channel_weights_follow_the_definition(oracle_mod):
    """Per-channel v weights with identity q, k: o of the first token from a zero state is
    beta (k.q) v'_0 with v'_0[c] = w[c][3] v_0[c] (rows before the start are zero)."""
    B, T, H, dk, dv = 1, 1, 2, 4, 6
    p = _inputs(B, T, H, dk, dv, seed=7)
    g = np.random.default_rng(8)
    wv = g.standard_normal((H * dv, 4)).astype(np.float32)
    r = oracle_mod.prefill_static(**p, wq=_onehot(H * dk, 3), wk=_onehot(H * dk, 3), wv=wv)
    for h in range(H):
        qh = p["q"][0, 0, h].astype(np.float64); kh = p["k"][0, 0, h].astype(np.float64)
        qh /= np.sqrt((qh ** 2).sum() + 1e-6); kh /= np.sqrt((kh ** 2).sum() + 1e-6)
        vc = wv[h * dv:(h + 1) * dv, 3].astype(np.float64) * p["v"][0, 0, h]
        np.testing.assert_allclose(r["o"][0, 0, h], p["beta"][0, 0, h] * (kh @ qh) * vc, rtol=1e-12, atol=1e-15)


def test_split_prefill_and_decode_loop(oracle_mod):
    B, T, H, dk, dv = 2, 12, 2, 4, 6
    p = _inputs(B, T, H, dk, dv, seed=9)
    g = np.random.default_rng(10)
    w = dict(wq=g.standard_normal((H * dk, 4)).astype(np.float32),
             wk=g.standard_normal((H * dk, 4)).astype(np.float32),
             wv=g.standard_normal((H * dv, 4)).astype(np.float32))
    full = oracle_mod.prefill_static(**p, **w)
    cut = 5
    a = oracle_mod.prefill_static(**{k: x[:, :cut] for k, x in p.items()}, **w)
    b = oracle_mod.prefill_static(**{k: x[:, cut:] for k, x in p.items()}, **w, S0=a["S_final"].astype(np.float32),
                                  cache_q=a["cache_q"], cache_k=a["cache_k"], cache_v=a["cache_v"])
    np.testing.assert_allclose(b["o"], full["o"][:, cut:], rtol=1e-6, atol=1e-6)
    S = None
    cq = ck = cv = None
    for t in range(T):
        d = oracle_mod.decode_step_static(S, cq, ck, cv, p["q"][:, t], p["k"][:, t], p["v"][:, t],
                                          p["alpha"][:, t], p["beta"][:, t], **w)
        np.testing.assert_allclose(d["o"], full["o"][:, t], rtol=1e-6, atol=1e-6)
        S, cq, ck, cv = d["S"].astype(np.float32), d["cache_q"], d["cache_k"], d["cache_v"]
    np.testing.assert_array_equal(cv, full["cache_v"])


def test_q_k_normalised_after_their_convolution(oracle_mod):
    """Scaling the q and k weights by 2 scales the convolved q and k by 2, which the L2
    normalisation after the convolution removes up to its eps = 1e-6 (relative changes of
    ~1e-6 here): o must not change beyond that (it would double if the normalisation came
    first)."""
    p = _inputs(B=1, T=7, H=2, dk=4, dv=6, seed=12)
    g = np.random.default_rng(13)
    w = dict(wq=g.standard_normal((8, 4)).astype(np.float32), wk=g.standard_normal((8, 4)).astype(np.float32),
             wv=g.standard_normal((12, 4)).astype(np.float32))
    r1 = oracle_mod.prefill_static(**p, **w)
    r2 = oracle_mod.prefill_static(**p, wq=2 * w["wq"], wk=2 * w["wk"], wv=w["wv"])
    np.testing.assert_allclose(r2["o"], r1["o"], rtol=1e-4, atol=1e-9)
