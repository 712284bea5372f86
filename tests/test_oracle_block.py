"""Pins of the recurrent-block oracle (linear layers, GeLU, merge, block).

The block composes the already-pinned RG-LRU oracle with three linear layers
and the GeLU merge (page "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid
Attention", "Non-Linear Multiplicative Gating with GeLU", and the listing's
RecurrentBlock).  Each test checks a part against something that does not come
from the oracle: values of the standard normal distribution, an exact
identity of GeLU, a library matrix product, zero and linearity properties,
causality, and the decode-step composition of the RG-LRU oracle.
"""
import math

import numpy as np
import scipy.special

import oracle

RNG = np.random.default_rng(777)


def _rglru(D, H, seed=3):
    rng = np.random.default_rng(seed)
    K = D // H
    import synth
    return dict(conv_w=rng.normal(0, 0.5, (D, 4)), conv_b=rng.normal(0, 0.1, D),
                W_a=rng.normal(0, 1 / math.sqrt(K), (H, K, K)), b_a=rng.normal(0, 0.3, D),
                W_x=rng.normal(0, 1 / math.sqrt(K), (H, K, K)), b_x=rng.normal(0, 0.3, D),
                Lambda=synth.lambda_from_uniform(rng.uniform(size=D)))


def _proj(dm, D, seed=4):
    rng = np.random.default_rng(seed)
    return (rng.normal(0, 1 / math.sqrt(dm), (D, dm)), rng.normal(0, 1 / math.sqrt(dm), (D, dm)),
            rng.normal(0, 1 / math.sqrt(D), (dm, D)))


def test_gelu_normal_cdf_values_and_identity():
    # GeLU(v) = v Phi(v): Phi(0) = 1/2, Phi(1) = 0.841344746068542948...,
    # Phi(2) = 0.977249868051820792... (standard normal table values)
    v = np.array([0.0, 1.0, -1.0, 2.0, -2.0])
    g = oracle.gelu(v)
    np.testing.assert_allclose(g, [0.0, 0.8413447460685429, -0.15865525393145705,
                                   2 * 0.9772498680518208, -2 * 0.022750131948179195],
                               rtol=1e-14, atol=1e-15)
    # Phi(v) + Phi(-v) = 1, so GeLU(v) - GeLU(-v) = v exactly in the reals
    w = RNG.normal(0, 3, 1000)
    np.testing.assert_allclose(oracle.gelu(w) - oracle.gelu(-w), w, rtol=0, atol=1e-14)
    # against scipy's normal CDF
    np.testing.assert_allclose(oracle.gelu(w), w * scipy.special.ndtr(w), rtol=1e-13, atol=1e-15)
    # slope 1/2 at zero, identity far right, zero far left
    e = 1e-6
    assert abs((oracle.gelu(np.array([e]))[0] - oracle.gelu(np.array([-e]))[0]) / (2 * e) - 0.5) < 1e-9
    assert abs(oracle.gelu(np.array([12.0]))[0] - 12.0) < 1e-15
    assert abs(oracle.gelu(np.array([-12.0]))[0]) < 1e-30


def test_linear_equals_library_matmul_with_out_in_storage():
    x = RNG.normal(size=(3, 5, 7))
    W = RNG.normal(size=(11, 7))   # [out][in]
    y = oracle.linear(x, W)
    assert y.shape == (3, 5, 11)
    np.testing.assert_allclose(y, np.einsum("btk,nk->btn", x, W), rtol=1e-13, atol=1e-13)
    # a transposed W would give a different result on a non-square W
    assert oracle.linear(x, np.eye(7)).shape == (3, 5, 7)
    np.testing.assert_array_equal(oracle.linear(x, np.eye(7)), x)


def test_merge_is_y_times_gelu():
    y = RNG.normal(size=200)
    g = RNG.normal(size=200)
    np.testing.assert_allclose(oracle.merge(y, g), y * g * scipy.special.ndtr(g), rtol=1e-13, atol=1e-15)


def test_block_zero_input_and_zero_branch():
    dm, D, H = 6, 8, 2
    p, (p1, p2, po) = _rglru(D, H), _proj(dm, D)
    out, hl, ho = oracle.block_fwd(np.zeros((2, 5, dm)), p1, p2, po, **p)
    np.testing.assert_array_equal(out, 0.0)   # GeLU(0) = 0 kills every output
    # a zero second branch gives zero output whatever the first does
    x = RNG.normal(size=(2, 5, dm))
    out, _, _ = oracle.block_fwd(x, p1, np.zeros_like(p2), po, **p)
    np.testing.assert_array_equal(out, 0.0)


def test_block_is_linear_in_output_projection_and_causal():
    dm, D, H = 6, 8, 2
    p, (p1, p2, po) = _rglru(D, H), _proj(dm, D)
    x = RNG.normal(size=(2, 9, dm))
    o1, _, _ = oracle.block_fwd(x, p1, p2, po, **p)
    po2 = RNG.normal(size=po.shape)
    o2, _, _ = oracle.block_fwd(x, p1, p2, po2, **p)
    o12, _, _ = oracle.block_fwd(x, p1, p2, po + 2.0 * po2, **p)
    np.testing.assert_allclose(o12, o1 + 2.0 * o2, rtol=1e-11, atol=1e-12)
    # changing the last tokens leaves earlier outputs untouched
    x2 = x.copy()
    x2[:, 6:] = RNG.normal(size=(2, 3, dm))
    o3, _, _ = oracle.block_fwd(x2, p1, p2, po, **p)
    np.testing.assert_array_equal(o3[:, :6], o1[:, :6])
    assert np.abs(o3[:, 6:] - o1[:, 6:]).max() > 1e-3


def test_block_prefill_equals_decode_steps():
    # the same block run token by token through the RG-LRU step oracle, with
    # the per-token linear layers and merge applied around it
    dm, D, H, B, T = 5, 8, 2, 2, 7
    p, (p1, p2, po) = _rglru(D, H), _proj(dm, D)
    x = RNG.normal(size=(B, T, dm))
    h0 = RNG.normal(size=(B, D))
    hist = RNG.normal(size=(B, 3, D))
    out, hl, ho = oracle.block_fwd(x, p1, p2, po, **p, h0=h0, hist_in=hist)
    h, hs = h0.copy(), hist.copy()
    for t in range(T):
        yt, hs, h = oracle.step(oracle.linear(x[:, t], p1), **p, hist=hs, h=h)
        zt = oracle.merge(yt, oracle.linear(x[:, t], p2))
        np.testing.assert_allclose(oracle.linear(zt, po), out[:, t], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(h, hl, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hs, ho, rtol=0, atol=0)
