"""Pins of the oracle's backward: central finite differences of the oracle's
own forward in double, plus linearity of the vector-Jacobian product.

L(theta) = <dy, y> + <dh_last, h_last>; step eps = 1e-6 max(1, |theta|).
Pass if |FD - analytic| <= 1e-6 max(|analytic|, RMS(analytic tensor)).

Slice reading of the 9B-width workload's finite-difference check ("T = 16,
D = 8"): that workload's seeded tensors restricted to batch 0, the first 16
tokens and head 0 (K = 256, so the gate arithmetic is unchanged), with
h0 ~ N(0, 1) to exercise dh0, and every entry tied to channels 0..7 perturbed.
The alternative reading, a standalone D = 8 problem with one 8x8 block, is
checked too.
"""
import numpy as np
import pytest

import oracle
import synth

FD_TOL = 1e-6


def _loss(prob, dy, dh_last):
    y, h_last, _ = oracle.fwd(prob["u"], prob["conv_w"], prob["conv_b"], prob["W_a"], prob["b_a"],
                              prob["W_x"], prob["b_x"], prob["Lambda"], h0=prob["h0"],
                              hist_in=prob.get("hist"))
    return float(np.sum(dy * y) + np.sum(dh_last * h_last))


def _analytic(prob, dy, dh_last):
    return oracle.bwd(prob["u"], prob["conv_w"], prob["conv_b"], prob["W_a"], prob["b_a"],
                      prob["W_x"], prob["b_x"], prob["Lambda"], dy, h0=prob["h0"],
                      hist_in=prob.get("hist"), dh_last=dh_last)


GRAD_OF = dict(u="du", conv_w="dconv_w", conv_b="dconv_b", W_a="dW_a", b_a="db_a",
               W_x="dW_x", b_x="db_x", Lambda="dLambda", h0="dh0")


def _check_fd(prob, dy, dh_last, entries):
    g = _analytic(prob, dy, dh_last)
    worst = 0.0
    for name, idx in entries:
        arr = prob[name]
        theta = arr[idx]
        eps = 1e-6 * max(1.0, abs(theta))
        arr[idx] = theta + eps
        lp = _loss(prob, dy, dh_last)
        arr[idx] = theta - eps
        lm = _loss(prob, dy, dh_last)
        arr[idx] = theta
        fd = (lp - lm) / (2 * eps)
        gt = g[GRAD_OF[name]]
        rms = float(np.sqrt(np.mean(gt * gt)))
        an = gt[idx]
        err = abs(fd - an) / max(abs(an), rms, 1e-300)
        worst = max(worst, err)
        assert err <= FD_TOL, (name, idx, fd, an, err)
    return worst


def _slice_problem():
    cfg = synth.FWD_BWD_9B
    K = cfg.K
    p = synth.make_params(cfg.idx, cfg.D, cfg.H, cfg.io)
    # batch 0, tokens < 16, head 0 of the 9B-width workload's seeded tensors
    u = synth.widen(synth.make_activation(cfg.idx, "u", (1, 16, cfg.D), cfg.io))[:, :, :K]
    dy = synth.widen(synth.make_activation(cfg.idx, "dy", (1, 16, cfg.D), cfg.io))[:, :, :K]
    prob = dict(u=np.ascontiguousarray(u),
                conv_w=synth.widen(p.conv_w)[:K].copy(), conv_b=synth.widen(p.conv_b)[:K].copy(),
                W_a=synth.widen(p.W_a)[:1].copy(), b_a=synth.widen(p.b_a)[:K].copy(),
                W_x=synth.widen(p.W_x)[:1].copy(), b_x=synth.widen(p.b_x)[:K].copy(),
                Lambda=synth.widen(p.Lambda)[:K].copy(),
                h0=synth.normal(synth.seed_for(cfg.idx, "h0"), 0, K).reshape(1, K))
    return prob, np.ascontiguousarray(dy)


def test_fd_slice_of_9b_workload():
    prob, dy = _slice_problem()
    dh_last = np.zeros((1, prob["u"].shape[2]))
    entries = [("u", (0, t, d)) for t in range(16) for d in range(8)]
    entries += [("conv_w", (d, k)) for d in range(8) for k in range(4)]
    entries += [(n, (d,)) for n in ("conv_b", "b_a", "b_x", "Lambda") for d in range(8)]
    entries += [(n, (0, o, j)) for n in ("W_a", "W_x") for o in range(8) for j in range(8)]
    entries += [("h0", (0, d)) for d in range(8)]
    _check_fd(prob, dy, dh_last, entries)


def test_fd_standalone_d8_with_history_and_final_state_grad():
    rng = np.random.default_rng(5)
    B, T, D = 2, 16, 8
    prob = dict(u=rng.normal(size=(B, T, D)), conv_w=rng.normal(0, 0.5, (D, 4)),
                conv_b=rng.normal(0, 0.1, D), W_a=rng.normal(0, 8 ** -0.5, (1, D, D)),
                b_a=rng.normal(0, 0.5, D), W_x=rng.normal(0, 8 ** -0.5, (1, D, D)),
                b_x=rng.normal(0, 0.5, D), Lambda=synth.lambda_from_uniform(rng.uniform(size=D)),
                h0=rng.normal(size=(B, D)), hist=rng.normal(size=(B, 3, D)))
    dy = rng.normal(size=(B, T, D))
    dh_last = rng.normal(size=(B, D))
    entries = []
    for name, arr in prob.items():
        if name == "hist":
            continue
        for idx in np.ndindex(arr.shape):
            entries.append((name, idx))
    _check_fd(prob, dy, dh_last, entries)


def test_vjp_is_linear_in_upstream_gradient():
    rng = np.random.default_rng(9)
    B, T, D, H = 2, 10, 16, 2
    K = D // H
    prob = dict(u=rng.normal(size=(B, T, D)), conv_w=rng.normal(0, 0.5, (D, 4)),
                conv_b=rng.normal(0, 0.1, D), W_a=rng.normal(0, K ** -0.5, (H, K, K)),
                b_a=np.zeros(D), W_x=rng.normal(0, K ** -0.5, (H, K, K)), b_x=np.zeros(D),
                Lambda=synth.lambda_from_uniform(rng.uniform(size=D)), h0=rng.normal(size=(B, D)))
    dy1, dy2 = rng.normal(size=(B, T, D)), rng.normal(size=(B, T, D))
    z = np.zeros((B, D))
    g1, g2 = _analytic(prob, dy1, z), _analytic(prob, dy2, z)
    g12 = _analytic(prob, 2.0 * dy1 - 3.0 * dy2, z)
    for k in g1:
        np.testing.assert_allclose(g12[k], 2.0 * g1[k] - 3.0 * g2[k], rtol=1e-10,
                                   atol=1e-12 * max(1.0, np.abs(g12[k]).max()))


def test_vjp_matches_directional_derivative():
    # <dy, J v> = <J^T dy, v> for a random direction v over all parameters
    rng = np.random.default_rng(11)
    B, T, D = 1, 12, 8
    prob = dict(u=rng.normal(size=(B, T, D)), conv_w=rng.normal(0, 0.5, (D, 4)),
                conv_b=rng.normal(0, 0.1, D), W_a=rng.normal(0, 0.35, (1, D, D)),
                b_a=rng.normal(0, 0.5, D), W_x=rng.normal(0, 0.35, (1, D, D)),
                b_x=rng.normal(0, 0.5, D), Lambda=synth.lambda_from_uniform(rng.uniform(size=D)),
                h0=rng.normal(size=(B, D)))
    dy = rng.normal(size=(B, T, D))
    dh = rng.normal(size=(B, D))
    g = _analytic(prob, dy, dh)
    v = {k: rng.normal(size=a.shape) for k, a in prob.items()}
    eps = 1e-6
    plus = {k: a + eps * v[k] for k, a in prob.items()}
    minus = {k: a - eps * v[k] for k, a in prob.items()}
    jv = (_loss(plus, dy, dh) - _loss(minus, dy, dh)) / (2 * eps)
    jtv = sum(float(np.sum(g[GRAD_OF[k]] * v[k])) for k in prob)
    assert abs(jv - jtv) <= 1e-6 * max(abs(jtv), 1.0)
