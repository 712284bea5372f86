"""Pins of the local-attention oracle (sliding-window MQA, prefill and ring
decode).

Sources: the wiki note "Griffin", section "Local Attention Path" (the window
N(t) = {i : t - w < i <= t} and the softmax-weighted sum of values), and the
page "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid Attention", sections
"Local Sliding-Window Multi-Query Attention (MQA)" (one key and value head for
all query heads) and "Bounding the Key-Value Cache Footprint" (a cache of at
most W positions, evicted ring-buffer fashion).  Each test checks the oracle
against something it does not compute itself: a library softmax over a banded
mask, closed forms (window 1, constant keys, two tokens), invariances of
softmax, and the decode ring against the prefill.
"""
import numpy as np
import scipy.special

import oracle

RNG = np.random.default_rng(2024)


def _inputs(B, T, Hq, dh, seed=0):
    r = np.random.default_rng(seed)
    return r.normal(size=(B, T, Hq, dh)), r.normal(size=(B, T, dh)), r.normal(size=(B, T, dh))


def test_equals_library_softmax_over_banded_mask():
    B, T, Hq, dh, W, sc = 2, 37, 3, 8, 5, 0.3
    q, k, v = _inputs(B, T, Hq, dh)
    o = oracle.attn_fwd(q, k, v, W, sc)
    t = np.arange(T)
    allowed = (t[None, :] <= t[:, None]) & (t[None, :] > t[:, None] - W)   # [t][i]
    for b in range(B):
        for h in range(Hq):
            s = sc * q[b, :, h, :] @ k[b].T
            s = np.where(allowed, s, -np.inf)
            p = scipy.special.softmax(s, axis=1)
            np.testing.assert_allclose(o[b, :, h, :], p @ v[b], rtol=1e-12, atol=1e-12)


def test_window_one_returns_own_value():
    q, k, v = _inputs(1, 9, 2, 4, seed=1)
    o = oracle.attn_fwd(q, k, v, 1, 1.0)
    np.testing.assert_allclose(o, np.repeat(v[:, :, None, :], 2, axis=2), rtol=0, atol=1e-15)


def test_two_tokens_closed_form():
    q = np.array([[[[0.7]], [[-1.3]]]])
    k = np.array([[[2.0], [0.5]]])
    v = np.array([[[3.0], [-4.0]]])
    o = oracle.attn_fwd(q, k, v, 2, 0.5)
    s0, s1 = 0.5 * -1.3 * 2.0, 0.5 * -1.3 * 0.5
    want1 = (np.exp(s0) * 3.0 + np.exp(s1) * -4.0) / (np.exp(s0) + np.exp(s1))
    assert abs(o[0, 0, 0, 0] - 3.0) < 1e-15
    assert abs(o[0, 1, 0, 0] - want1) < 1e-14


def test_constant_keys_average_the_window():
    B, T, Hq, dh, W = 1, 20, 2, 6, 7
    q, _, v = _inputs(B, T, Hq, dh, seed=3)
    k = np.tile(RNG.normal(size=(1, 1, dh)), (B, T, 1))
    o = oracle.attn_fwd(q, k, v, W, 0.8)
    for t in range(T):
        lo = max(0, t - W + 1)
        np.testing.assert_allclose(o[0, t], np.tile(v[0, lo:t + 1].mean(axis=0), (Hq, 1)), rtol=1e-12,
                                   atol=1e-13)


def test_window_at_least_t_is_causal_attention_and_shift_invariant():
    q, k, v = _inputs(2, 16, 2, 5, seed=4)
    o16 = oracle.attn_fwd(q, k, v, 16, 0.4)
    np.testing.assert_allclose(oracle.attn_fwd(q, k, v, 1000, 0.4), o16, rtol=0, atol=0)
    # adding one vector to every key shifts each row's scores by a constant
    c = RNG.normal(size=5)
    np.testing.assert_allclose(oracle.attn_fwd(q, k + c, v, 16, 0.4), o16, rtol=1e-11, atol=1e-12)
    # and the shorter window differs from it once t >= W
    o4 = oracle.attn_fwd(q, k, v, 4, 0.4)
    np.testing.assert_allclose(o4[:, :4], o16[:, :4], rtol=0, atol=0)
    assert np.max(np.abs(o4[:, 4:] - o16[:, 4:])) > 1e-3


def test_query_heads_share_one_key_value_head():
    q, k, v = _inputs(1, 12, 3, 4, seed=5)
    q[:, :, 2] = q[:, :, 0]
    o = oracle.attn_fwd(q, k, v, 6, 0.7)
    np.testing.assert_array_equal(o[:, :, 2], o[:, :, 0])
    # each head alone gives the same as within the group
    o1 = oracle.attn_fwd(np.ascontiguousarray(q[:, :, 1:2]), k, v, 6, 0.7)
    np.testing.assert_allclose(o1[:, :, 0], o[:, :, 1], rtol=0, atol=0)


def test_ring_decode_equals_prefill_past_the_window():
    # T > W so the ring wraps and evicts; streams start at different positions
    B, T, Hq, dh, W, sc = 2, 23, 2, 4, 6, 0.5
    q, k, v = _inputs(B, T, Hq, dh, seed=6)
    ref = oracle.attn_fwd(q, k, v, W, sc)
    kc = np.full((B, W, dh), np.nan)   # never-written slots must not be read
    vc = np.full((B, W, dh), np.nan)
    for t in range(T):
        o = oracle.attn_step(np.ascontiguousarray(q[:, t]), np.ascontiguousarray(k[:, t]),
                             np.ascontiguousarray(v[:, t]), kc, vc, np.full(B, t), sc)
        np.testing.assert_allclose(o, ref[:, t], rtol=1e-13, atol=1e-13)
    # the ring holds the last W positions, position p in slot p mod W
    for p in range(T - W, T):
        np.testing.assert_array_equal(kc[:, p % W], k[:, p])
