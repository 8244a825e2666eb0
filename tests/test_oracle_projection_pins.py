"""CPU pins of the oracle's input projections (jbo_project, prefill_from_x):
bf16 rounding against an independent implementation and hand-computed ties,
one-hot inputs that expose the weight orientation, closed-form gates, and the
composition with the block."""
import math

import numpy as np
import pytest
import torch


@pytest.fixture(scope="module")
def oracle_mod():
    import oracle
    oracle.build()
    return oracle


def test_bf16_round_hand_values(oracle_mod):
    r = oracle_mod.bf16_round
    assert r(1.0 + 2.0 ** -8) == 1.0                            # halfway: ties to the even 1.0
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6            # halfway: ties to the even mantissa
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7   # just above halfway
    assert r(-(1.0 + 2.0 ** -8)) == -1.0
    assert r(3 * 2.0 ** -134) == 2.0 ** -132                    # subnormal spacing 2^-133, tie to even
    assert r(0.0) == 0.0 and r(255.5) == 256.0 and r(254.5) == 254.0


def test_bf16_round_matches_torch_on_float32_values(oracle_mod):
    """torch's float32 -> bfloat16 conversion (round to nearest even) is an independent
    implementation; on float32 inputs both must agree exactly."""
    g = np.random.default_rng(5)
    vals = np.concatenate([g.standard_normal(2000) * 10.0 ** g.integers(-30, 30, 2000),
                           (1.0 + (2 * g.integers(0, 128, 200) + 1) * 2.0 ** -8)]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.bfloat16).float().numpy()
    got = np.array([oracle_mod.bf16_round(float(v)) for v in vals], np.float32)
    np.testing.assert_array_equal(got, ref)


def _proj_inputs(B=1, T=3, D=8, H=2, dk=3, dv=4, seed=0):
    g = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy()
    return dict(x=bf(g.standard_normal((B, T, D))), Wq=bf(g.standard_normal((H * dk, D)) * 0.3),
                Wk=bf(g.standard_normal((H * dk, D)) * 0.3), Wv=bf(g.standard_normal((H * dv, D)) * 0.3),
                Wa=bf(g.standard_normal((H, D)) * 0.3), Wb=bf(g.standard_normal((H, D)) * 0.3))


def test_one_hot_inputs_read_weight_columns(oracle_mod):
    """x = e_i makes q[r] the weight entry Wq[r, i] (rounded to bf16), for non-square weights:
    a transposed weight or a wrong row stride cannot pass."""
    p = _proj_inputs(T=8, D=8, H=2, dk=3, dv=5)
    p["x"] = np.eye(8, dtype=np.float32)[None]                   # token t = e_t
    r = oracle_mod.project(**p)
    for t in range(8):
        np.testing.assert_array_equal(r["q"][0, t].reshape(-1), p["Wq"][:, t])
        np.testing.assert_array_equal(r["k"][0, t].reshape(-1), p["Wk"][:, t])
        np.testing.assert_array_equal(r["v"][0, t].reshape(-1), p["Wv"][:, t])
        np.testing.assert_allclose(r["alpha"][0, t], 1.0 / (1.0 + np.exp(-p["Wa"][:, t].astype(np.float64))),
                                   rtol=1e-15)


def test_rounding_happens_after_the_exact_sum(oracle_mod):
    """q = 1 + 2^-8 exactly is a bf16 tie (-> 1.0); adding 2^-30 tips it to 1 + 2^-7.  A
    projection that rounded the products, or accumulated in float32 (24 bits: 1 + 2^-8 +
    2^-30 is 1 + 2^-8 there) before rounding, would not see the 2^-30."""
    x = np.array([[[1.0, 2.0 ** -8, 2.0 ** -30]]], np.float32)
    W = np.array([[1.0, 1.0, 0.0], [1.0, 1.0, 1.0]], np.float32)   # H=1, dk=2
    Wv = np.array([[1.0, 1.0, 1.0]], np.float32)
    Z = np.zeros((1, 3), np.float32)
    r = oracle_mod.project(x, W, W, Wv, Z, Z)
    assert r["q"][0, 0, 0].tolist() == [1.0, 1.0 + 2.0 ** -7]
    assert r["v"][0, 0, 0, 0] == 1.0 + 2.0 ** -7


def test_gates_closed_form_and_biases(oracle_mod):
    p = _proj_inputs(H=3)
    H, D = 3, p["x"].shape[2]
    Z = np.zeros((H, D), np.float32)
    ba = np.array([-2.0, 0.0, 3.5], np.float32)
    bb = np.array([0.25, -1.0, 8.0], np.float32)
    r = oracle_mod.project(p["x"], p["Wq"][:9], p["Wk"][:9], p["Wv"][:12], Z, Z, ba=ba, bb=bb)
    for h in range(H):
        assert r["alpha"][0, :, h] == pytest.approx(1.0 / (1.0 + math.exp(-float(ba[h]))), rel=1e-15)
        assert r["beta"][0, :, h] == pytest.approx(1.0 / (1.0 + math.exp(-float(bb[h]))), rel=1e-15)
    # a bias on q shifts q by exactly that bias when Wq is zero
    bq = np.arange(9, dtype=np.float32) - 4.0
    r2 = oracle_mod.project(p["x"], np.zeros((9, D), np.float32), p["Wk"][:9], p["Wv"][:12], Z, Z, bq=bq)
    np.testing.assert_array_equal(r2["q"][0, 0].reshape(-1), bq)


def test_projections_scale_exactly_by_powers_of_two(oracle_mod):
    p = _proj_inputs(T=5)
    r1 = oracle_mod.project(**p)
    p2 = dict(p, x=p["x"] * 4.0)
    r2 = oracle_mod.project(**p2)
    for key in ("q", "k", "v"):
        np.testing.assert_array_equal(r2[key], 4.0 * r1[key])


def test_prefill_from_x_is_projection_then_block(oracle_mod):
    """The composed oracle equals the block run on the projections' outputs, and with
    one-hot selecting weights the block sees slices of x itself."""
    g = np.random.default_rng(3)
    B, T, H, dk, dv, D = 1, 9, 2, 2, 4, 16
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy()
    x = bf(g.standard_normal((B, T, D)))
    sel = lambda rows, off: np.eye(D, dtype=np.float32)[off:off + rows]
    Wq, Wk, Wv = sel(H * dk, 0), sel(H * dk, 4), sel(H * dv, 8)
    Wa, Wb = bf(g.standard_normal((H, D)) * 0.2), bf(g.standard_normal((H, D)) * 0.2)
    W1, W2 = bf(g.standard_normal((32, D)) * 0.1), bf(g.standard_normal((4 * H, 32)) * 0.1)
    r = oracle_mod.prefill_from_x(x, Wq, Wk, Wv, Wa, Wb, W1, W2)
    q = x[:, :, 0:4].reshape(B, T, H, dk)
    k = x[:, :, 4:8].reshape(B, T, H, dk)
    v = x[:, :, 8:16].reshape(B, T, H, dv)
    np.testing.assert_array_equal(r["proj"]["q"], q)
    np.testing.assert_array_equal(r["proj"]["v"], v)
    a = (1.0 / (1.0 + np.exp(-np.einsum("btd,hd->bth", x.astype(np.float64), Wa.astype(np.float64))))).astype(np.float32)
    b = (1.0 / (1.0 + np.exp(-np.einsum("btd,hd->bth", x.astype(np.float64), Wb.astype(np.float64))))).astype(np.float32)
    ref = oracle_mod.prefill(x, q, k, v, a, b, W1, W2)
    np.testing.assert_allclose(r["o"], ref["o"], rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(r["S_final"], ref["S_final"], rtol=1e-6, atol=1e-9)
