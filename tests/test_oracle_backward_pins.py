"""CPU pins of the oracle's backward pass (jbo_backward) against things it does not compute
itself: central differences of the pinned forward oracle along random directions for every
input, across the 64-token checkpoint, a closed form with beta = 0, linearity in the output
gradients, and thread-count independence."""
import numpy as np
import pytest


@pytest.fixture(scope="module")
def oracle_mod():
    import oracle
    oracle.build()
    return oracle


NAMES = {"x": "dx", "q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "beta": "dbeta", "W1": "dW1", "b1": "db1",
         "W2": "dW2", "b2": "db2", "S0": "dS0", "conv_in": "dconv_in"}
# inputs the loss depends on linearly: central differences are exact up to rounding
LINEAR = {"v", "W2", "b2", "S0", "conv_in"}


def _case(B, T, H, dk, dv, D, seed):
    g = np.random.default_rng(seed)
    f = lambda *s: g.standard_normal(s)
    p = dict(x=f(B, T, D), q=f(B, T, H, dk), k=f(B, T, H, dk), v=f(B, T, H, dv),
             alpha=0.5 + 0.45 * g.random((B, T, H)), beta=g.random((B, T, H)), W1=0.3 * f(32, D),
             W2=0.3 * f(4 * H, 32), b1=0.1 * f(32), b2=0.1 * f(4 * H), S0=0.3 * f(B, H, dk, dv),
             conv_in=f(B, 3, H, dv))
    p = {k: v.astype(np.float32) for k, v in p.items()}
    grads = dict(dout=f(B, T, H, dv).astype(np.float32), dS_final=f(B, H, dk, dv).astype(np.float32),
                 dconv_out=f(B, 3, H, dv).astype(np.float32))
    return p, grads, g


def _loss(oracle_mod, p, grads):
    r = oracle_mod.prefill(p["x"], p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["W1"], p["W2"], b1=p["b1"],
                           b2=p["b2"], S0=p["S0"], conv_in=p["conv_in"])
    return float((r["o"] * grads["dout"]).sum() + (r["S_final"] * grads["dS_final"]).sum()
                 + (r["conv_out"].astype(np.float64) * grads["dconv_out"]).sum())


def _fd_check(oracle_mod, p, grads, g, names, eps=2e-4):
    r = oracle_mod.backward(**p, **grads)
    for n in names:
        d = g.standard_normal(p[n].shape)
        pp, pm = dict(p), dict(p)
        pp[n] = (p[n] + eps * d).astype(np.float32)
        pm[n] = (p[n] - eps * d).astype(np.float32)
        step = pp[n].astype(np.float64) - pm[n].astype(np.float64)   # the exact float32 step taken
        fd = _loss(oracle_mod, pp, grads) - _loss(oracle_mod, pm, grads)
        an = float((r[NAMES[n]] * step).sum())
        rel = abs(fd - an) / max(abs(an), 1e-300)
        tol = 1e-9 if n in LINEAR else 2e-5   # eps^2 truncation for the nonlinear inputs
        print(f"  {n}: fd {fd:.6e} analytic {an:.6e} rel {rel:.1e}", flush=True)
        assert rel < tol, (n, fd, an, rel)


def test_every_gradient_against_central_differences(oracle_mod):
    p, grads, g = _case(2, 7, 2, 4, 6, 8, seed=0)
    _fd_check(oracle_mod, p, grads, g, list(NAMES))


def test_gradients_across_the_checkpoint(oracle_mod):
    """150 tokens: the reverse pass recomputes states from checkpoints every 64 tokens."""
    p, grads, g = _case(1, 150, 1, 4, 5, 8, seed=1)
    _fd_check(oracle_mod, p, grads, g, ["k", "alpha", "beta", "S0", "v"])


def test_beta_zero_closed_form(oracle_mod):
    """beta = 0, alpha = 1: the state never changes, o_t = S0^T q^_t, so dS0 = dS_final +
    sum_t q^_t do_t^T, and no gradient reaches v, alpha or k."""
    p, grads, g = _case(1, 9, 2, 4, 6, 8, seed=2)
    p["beta"][:] = 0.0
    p["alpha"][:] = 1.0
    grads["dconv_out"] = None
    r = oracle_mod.backward(**p, **grads)
    qh = p["q"].astype(np.float64)
    qh = qh / np.sqrt((qh ** 2).sum(-1, keepdims=True) + 1e-6)
    want = grads["dS_final"].astype(np.float64) + np.einsum("bthi,bthc->bhic", qh, grads["dout"].astype(np.float64))
    np.testing.assert_allclose(r["dS0"], want, rtol=1e-12, atol=1e-12)
    assert np.all(r["dv"] == 0) and np.all(r["dk"] == 0) and np.all(r["dconv_in"] == 0)
    # dalpha_t = sum(dM_t . S0) with dM_t the gradient flowing into M_t
    assert np.all(np.isfinite(r["dalpha"]))


def test_linear_in_the_output_gradients(oracle_mod):
    p, g1, g = _case(1, 20, 2, 4, 6, 8, seed=3)
    _, g2, _ = _case(1, 20, 2, 4, 6, 8, seed=4)
    # multiples of 2^-10: g1 + 2 g2 is then exact in float32
    g1 = {k: (np.round(v * 1024) / 1024).astype(np.float32) for k, v in g1.items()}
    g2 = {k: (np.round(v * 1024) / 1024).astype(np.float32) for k, v in g2.items()}
    r1 = oracle_mod.backward(**p, **g1)
    r2 = oracle_mod.backward(**p, **g2)
    g12 = {k: (g1[k].astype(np.float64) + 2 * g2[k].astype(np.float64)).astype(np.float32) for k in g1}
    r12 = oracle_mod.backward(**p, **g12)
    for n in NAMES.values():
        np.testing.assert_allclose(r12[n], r1[n] + 2 * r2[n], rtol=1e-10, atol=1e-12 * np.abs(r12[n]).max(),
                                   err_msg=n)


def test_thread_count_independence(oracle_mod):
    p, grads, _ = _case(2, 30, 3, 4, 6, 8, seed=5)
    r1 = oracle_mod.backward(**p, **grads, nthreads=1)
    r4 = oracle_mod.backward(**p, **grads, nthreads=4)
    for n in NAMES.values():
        assert np.array_equal(r1[n], r4[n]), n
