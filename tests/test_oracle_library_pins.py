"""Pins of the oracle against independent library implementations.

Each check compares an oracle function with a routine that was written
elsewhere and ships in this image, so that a mistake in the oracle that its
own identities could miss (a wrong exponent, a dropped constant, a transposed
operand) fails here:

- RG-LRU core (page "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid
  Attention", "Formulation of the RG-LRU Gating Mechanism"): the
  RecurrentGemma RG-LRU layer of the `transformers` package, run in float64.
  That layer stores its gate weights [in][out] (x @ W), parametrises the
  decay with softplus of its own parameter (log a = -8 r softplus(p), so
  p = -Lambda here) and resets the state at position 0; positions that start
  at 1 switch the reset off, which leaves the pages' update
  h_t = a_t h_{t-1} + sqrt(1 - a_t^2) i_t x_t.  Its scan rounds the decay to
  float32, hence the 1e-6 tolerance.
- Rotary embedding (same page, "Local Sliding-Window Multi-Query Attention
  (MQA)": standard RoPE on queries and keys): the rotary helpers of the
  `transformers` Llama model (half-split pairs (j, j + dh/2), frequency
  base^(-2j/dh)), and a value worked by hand for a pair j >= 1.
- GELU, tanh form (module page
  "transformer_lens.model_bridge.supported_architectures.recurrent_gemma",
  "Architecture overview"): torch's gelu(approximate="tanh") in float64, at
  points where the cubic term moves the value by far more than the tolerance.
"""
import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(2024)


def _rglru_module(D, H):
    from transformers.models.recurrent_gemma.configuration_recurrent_gemma import RecurrentGemmaConfig
    from transformers.models.recurrent_gemma.modeling_recurrent_gemma import RecurrentGemmaRglru
    cfg = RecurrentGemmaConfig(lru_width=D, num_attention_heads=H, hidden_size=D)
    return RecurrentGemmaRglru(cfg).double()


@pytest.mark.parametrize("B,T,D,H", [(2, 9, 16, 2), (1, 40, 24, 3)])
def test_rglru_core_against_transformers_recurrentgemma(B, T, D, H):
    pytest.importorskip("transformers")
    K = D // H
    x = RNG.normal(size=(B, T, D))
    W_a = RNG.normal(0, K ** -0.5, (H, K, K))
    W_x = RNG.normal(0, K ** -0.5, (H, K, K))
    b_a = RNG.normal(0, 0.5, D)
    b_x = RNG.normal(0, 0.5, D)
    lam = np.log(np.power(RNG.uniform(0.9, 0.999, D), 1 / 8) / (1 - np.power(RNG.uniform(0.9, 0.999, D), 1 / 8)))
    lam[:3] = (-2.0, 0.5, 3.0)   # a few decays far from the initialiser's range
    h0 = RNG.normal(size=(B, D))

    m = _rglru_module(D, H)
    with torch.no_grad():
        m.recurrent_param.copy_(torch.from_numpy(-lam))
        m.input_gate_weight.copy_(torch.from_numpy(W_x.transpose(0, 2, 1).copy()))
        m.recurrent_gate_weight.copy_(torch.from_numpy(W_a.transpose(0, 2, 1).copy()))
        m.input_gate_bias.copy_(torch.from_numpy(b_x.reshape(H, K)))
        m.recurrent_gate_bias.copy_(torch.from_numpy(b_a.reshape(H, K)))
        m.recurrent_states = torch.from_numpy(h0.copy())
        pos = torch.arange(1, T + 1).expand(B, T)
        ref = m(torch.from_numpy(x), pos).numpy()

    r, i = oracle.gates(x, W_a, b_a, W_x, b_x)
    y, h_last = oracle.scan(x, r, i, lam, h0)
    assert oracle.rel_err(y, ref) < 1e-6
    assert oracle.rel_err(h_last, ref[:, -1]) < 1e-6
    # the same layer with its gate weights used the other way round disagrees
    # (the pin sees a transposed W)
    r2, i2 = oracle.gates(x, W_a.transpose(0, 2, 1).copy(), b_a, W_x.transpose(0, 2, 1).copy(), b_x)
    y2, _ = oracle.scan(x, r2, i2, lam, h0)
    assert oracle.rel_err(y2, ref) > 1e-3


def test_rope_pair_above_zero_by_hand():
    # base 4, rot 4: pair j = 1 is (1, 3) and turns by p * 4^(-2/4) = p / 2;
    # at position 2 that is exactly 1 rad
    e = np.zeros((1, 1, 4))
    e[0, 0, 1] = 1.0
    r = oracle.rope(e, np.array([2]), 4, base=4.0)
    assert abs(r[0, 0, 1] - math.cos(1.0)) < 1e-15
    assert abs(r[0, 0, 3] - math.sin(1.0)) < 1e-15
    assert r[0, 0, 0] == 0.0 and r[0, 0, 2] == 0.0
    # pair j = 0 at the same position turns by 2 rad
    e = np.zeros((1, 1, 4))
    e[0, 0, 2] = 1.0   # second member of pair 0
    r = oracle.rope(e, np.array([2]), 4, base=4.0)
    assert abs(r[0, 0, 0] + math.sin(2.0)) < 1e-15 and abs(r[0, 0, 2] - math.cos(2.0)) < 1e-15


@pytest.mark.parametrize("dh,base", [(16, 10000.0), (64, 500.0)])
def test_rope_against_transformers_llama_rotary(dh, base):
    pytest.importorskip("transformers")
    from transformers.models.llama.modeling_llama import rotate_half
    H, M = 3, 7
    x = RNG.normal(size=(M, H, dh))
    pos = np.array([0, 1, 5, 17, 250, 4095, 70000])
    # the Llama rotary embedding's tables: inv_freq = base^(-2j/dh), angle
    # pos * inv_freq duplicated over both halves, x cos + rotate_half(x) sin
    inv = 1.0 / (base ** (torch.arange(0, dh, 2, dtype=torch.float64) / dh))
    ang = torch.from_numpy(pos).double()[:, None] * inv[None, :]
    emb = torch.cat([ang, ang], dim=-1)[:, None, :]
    xt = torch.from_numpy(x)
    ref = (xt * emb.cos() + rotate_half(xt) * emb.sin()).numpy()
    got = oracle.rope(x, pos, dh, base=base)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-9)


def test_gelu_tanh_against_torch_tanh_approximation():
    v = np.concatenate([RNG.normal(0, 2, 500), np.array([-3.0, -1.0, -0.5, 0.5, 1.0, 1.5, 2.0, 3.0])])
    ref = torch.nn.functional.gelu(torch.from_numpy(v), approximate="tanh").numpy()
    got = oracle.gelu_tanh(v)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)
    # at v = 1.5 the cubic term moves the value by ~2.7e-2; a wrong coefficient shows
    no_cubic = 0.5 * 1.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * 1.5))
    assert abs(oracle.gelu_tanh(np.array([1.5]))[0] - no_cubic) > 1e-2
