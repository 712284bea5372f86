"""Pins of the residual-layer oracle (RMSNorm, GELU-tanh, gated MLP, the Hawk
layer with the recurrent block as temporal mixer).

Sources: the wiki note "Griffin", section "Residual Block View" (pre-norm
residual scaffold), and the module page
"transformer_lens.model_bridge.supported_architectures.recurrent_gemma",
"Architecture overview" (temporal and channel pre-norms, gated MLP with
GELU-tanh, RMSNorm applying 1 + weight).  Checks use what the oracle does not
compute itself: norms and invariances, values and limits of the tanh form
against the exact GeLU, library matrix products, and the layer's reductions
to identity and to the already-pinned block.
"""
import math

import numpy as np

import oracle

RNG = np.random.default_rng(99)


def test_rmsnorm_unit_rms_scale_invariance_and_weight():
    x = RNG.normal(0, 3, (7, 64))
    y = oracle.rmsnorm(x, np.zeros(64), eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.rmsnorm(5.0 * x, np.zeros(64), eps=0.0), y, rtol=1e-14)
    w = RNG.normal(size=64)
    np.testing.assert_allclose(oracle.rmsnorm(x, w, eps=0.0), y * (1.0 + w), rtol=1e-14)
    # eps enters under the root: a zero row stays zero, a tiny row is damped
    z = oracle.rmsnorm(np.zeros((1, 64)), np.zeros(64), eps=1e-6)
    assert np.all(z == 0.0)
    t = oracle.rmsnorm(np.full((1, 64), 1e-3), np.zeros(64), eps=1e-6)
    np.testing.assert_allclose(t, 1e-3 / math.sqrt(1e-6 + 1e-6), rtol=1e-14)


def test_gelu_tanh_identity_limits_and_distance_to_exact_gelu():
    v = RNG.normal(0, 3, 2000)
    g = oracle.gelu_tanh(v)
    # tanh is odd, so GELU_tanh(v) - GELU_tanh(-v) = v exactly in the reals
    np.testing.assert_allclose(g - oracle.gelu_tanh(-v), v, rtol=0, atol=1e-13)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert abs(oracle.gelu_tanh(np.array([10.0]))[0] - 10.0) < 1e-12
    assert abs(oracle.gelu_tanh(np.array([-10.0]))[0]) < 1e-12
    # slope 1/2 at 0 (the cubic term is third order)
    e = 1e-6
    assert abs((oracle.gelu_tanh(np.array([e]))[0] - oracle.gelu_tanh(np.array([-e]))[0]) / (2 * e) - 0.5) < 1e-9
    # a close approximation of the exact (erf) GeLU, the tanh form's purpose
    d = np.max(np.abs(g - oracle.gelu(v)))
    assert 1e-5 < d < 1e-3


def test_mlp_against_library_products():
    x = RNG.normal(size=(2, 5, 12))
    gw, uw, dw = RNG.normal(size=(20, 12)), RNG.normal(size=(20, 12)), RNG.normal(size=(12, 20))
    out = oracle.mlp(x, gw, uw, dw)
    a = np.einsum("btk,nk->btn", x, gw)
    b = np.einsum("btk,nk->btn", x, uw)
    np.testing.assert_allclose(out, np.einsum("btf,df->btd", oracle.gelu_tanh(a) * b, dw), rtol=1e-12, atol=1e-12)
    # linear in down, zero when up is zero
    np.testing.assert_allclose(oracle.mlp(x, gw, uw, 3 * dw), 3 * out, rtol=1e-13)
    assert np.all(oracle.mlp(x, gw, np.zeros_like(uw), dw) == 0.0)


def _layer_params(dm, D, F, seed=5):
    r = np.random.default_rng(seed)
    import synth
    return dict(tnorm_w=r.normal(0, 0.1, dm), cnorm_w=r.normal(0, 0.1, dm),
                proj_in_1=r.normal(0, dm ** -0.5, (D, dm)), proj_in_2=r.normal(0, dm ** -0.5, (D, dm)),
                proj_out=r.normal(0, D ** -0.5, (dm, D)), conv_w=r.normal(0, 0.5, (D, 4)), conv_b=r.normal(0, 0.1, D),
                W_a=r.normal(0, D ** -0.5, (1, D, D)), b_a=r.normal(0, 0.3, D),
                W_x=r.normal(0, D ** -0.5, (1, D, D)), b_x=r.normal(0, 0.3, D),
                Lambda=synth.lambda_from_uniform(r.uniform(size=D)),
                gate_w=r.normal(0, dm ** -0.5, (F, dm)), up_w=r.normal(0, dm ** -0.5, (F, dm)),
                down_w=r.normal(0, F ** -0.5, (dm, F)))


def test_layer_reduces_to_identity_and_to_the_block():
    dm, D, F = 24, 16, 40
    p = _layer_params(dm, D, F)
    x = RNG.normal(size=(2, 9, dm))
    zero = dict(p, proj_out=np.zeros_like(p["proj_out"]), down_w=np.zeros_like(p["down_w"]))
    y, _, _ = oracle.hawk_layer(x, **zero)
    np.testing.assert_array_equal(y, x)
    # MLP off: x + block(RMSNorm(x)) with the pinned block oracle
    y1, h1, s1 = oracle.hawk_layer(x, **dict(p, down_w=np.zeros_like(p["down_w"])))
    bp = {k: p[k] for k in ("proj_in_1", "proj_in_2", "proj_out", "conv_w", "conv_b", "W_a", "b_a", "W_x", "b_x",
                            "Lambda")}
    t, h2, s2 = oracle.block_fwd(oracle.rmsnorm(x, p["tnorm_w"]), **bp)
    np.testing.assert_allclose(y1, x + t, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(h1, h2)
    # temporal mixer off: x + MLP(RMSNorm(x))
    y2, _, _ = oracle.hawk_layer(x, **dict(p, proj_out=np.zeros_like(p["proj_out"])))
    np.testing.assert_allclose(y2, x + oracle.mlp(oracle.rmsnorm(x, p["cnorm_w"]), p["gate_w"], p["up_w"],
                                                  p["down_w"]), rtol=1e-14, atol=1e-14)


def test_layer_is_causal_and_splits_with_state():
    dm, D, F = 20, 16, 32
    p = _layer_params(dm, D, F, seed=6)
    x = RNG.normal(size=(1, 30, dm))
    y, h, s = oracle.hawk_layer(x, **p)
    x2 = x.copy()
    x2[:, 20:] += RNG.normal(size=(1, 10, dm))
    y2, _, _ = oracle.hawk_layer(x2, **p)
    np.testing.assert_array_equal(y2[:, :20], y[:, :20])
    ya, ha, sa = oracle.hawk_layer(x[:, :13], **p)
    yb, hb, _ = oracle.hawk_layer(x[:, 13:], **p, h0=ha, hist_in=sa)
    np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hb, h, rtol=1e-12, atol=1e-12)
