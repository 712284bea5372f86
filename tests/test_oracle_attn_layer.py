"""Pins of the rotary embedding and the attention residual layer oracle.

Sources: the page "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid Attention",
"Local Sliding-Window Multi-Query Attention (MQA)" (standard rotary position
embeddings on queries and keys), the module page
"transformer_lens.model_bridge.supported_architectures.recurrent_gemma"
(q/k/v/o projections, partial rotary), and the wiki note "Griffin", "Residual
Block View".  Checks: rotations keep norms, the score of a rotated query and
key depends only on the positions' difference, position 0 and rot = 0 are
the identity, dimensions past rot are untouched, a hand-computed rotation;
and the layer is invariant to a shift of all positions, reduces to x + MLP
when the output projection is zero, and is causal.
"""
import math

import numpy as np

import oracle

RNG = np.random.default_rng(31)


def test_rope_rotation_properties():
    x = RNG.normal(size=(5, 3, 16))
    pos = np.array([0, 1, 7, 100, 5000])
    y = oracle.rope(x, pos, 16)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(y[0], x[0], rtol=0, atol=0)                 # position 0
    np.testing.assert_array_equal(oracle.rope(x, pos, 0), x)               # rot = 0
    z = oracle.rope(x, pos, 8)                                             # partial: dims >= 8 untouched
    np.testing.assert_array_equal(z[..., 8:], x[..., 8:])
    # hand-computed: pair (0, 4) of a rot = 8 head at position 3 turns by 3 rad
    e = np.zeros((1, 1, 8)); e[0, 0, 0] = 1.0
    r = oracle.rope(e, np.array([3]), 8)
    assert abs(r[0, 0, 0] - math.cos(3.0)) < 1e-15 and abs(r[0, 0, 4] - math.sin(3.0)) < 1e-15


def test_rope_scores_depend_on_relative_position_only():
    q = RNG.normal(size=(1, 1, 32))
    k = RNG.normal(size=(1, 1, 32))
    def score(m, n):
        return float(np.sum(oracle.rope(q, np.array([m]), 32) * oracle.rope(k, np.array([n]), 32)))
    for m, n in ((5, 2), (40, 37), (1000, 997)):
        assert abs(score(m, n) - score(5, 2)) < 1e-10


def _params(dm, Hq, dh, F, seed=8):
    r = np.random.default_rng(seed)
    return dict(tnorm_w=r.normal(0, 0.1, dm), cnorm_w=r.normal(0, 0.1, dm),
                wq=r.normal(0, dm ** -0.5, (Hq * dh, dm)), wk=r.normal(0, dm ** -0.5, (dh, dm)),
                wv=r.normal(0, dm ** -0.5, (dh, dm)), wo=r.normal(0, (Hq * dh) ** -0.5, (dm, Hq * dh)),
                gate_w=r.normal(0, dm ** -0.5, (F, dm)), up_w=r.normal(0, dm ** -0.5, (F, dm)),
                down_w=r.normal(0, F ** -0.5, (dm, F)))


def test_attention_layer_shift_invariance_reduction_and_causality():
    dm, Hq, dh, F, W = 24, 3, 8, 40, 5
    p = _params(dm, Hq, dh, F)
    x = RNG.normal(size=(2, 12, dm))
    y = oracle.attn_layer(x, **p, Hq=Hq, window=W, scale=dh ** -0.5, rot=dh)
    # scores depend on position differences only: shifting every position changes nothing
    np.testing.assert_allclose(oracle.attn_layer(x, **p, Hq=Hq, window=W, scale=dh ** -0.5, rot=dh, pos0=777),
                               y, rtol=1e-10, atol=1e-11)
    # output projection off: x + MLP(RMSNorm(x))
    y0 = oracle.attn_layer(x, **dict(p, wo=np.zeros_like(p["wo"])), Hq=Hq, window=W, scale=0.3, rot=dh)
    np.testing.assert_allclose(y0, x + oracle.mlp(oracle.rmsnorm(x, p["cnorm_w"]), p["gate_w"], p["up_w"],
                                                  p["down_w"]), rtol=1e-14, atol=1e-14)
    # causal
    x2 = x.copy()
    x2[:, 8:] += 1.0
    np.testing.assert_array_equal(oracle.attn_layer(x2, **p, Hq=Hq, window=W, scale=dh ** -0.5, rot=dh)[:, :8],
                                  y[:, :8])
