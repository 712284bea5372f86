"""GPU parity of the attention residual layer (rglru_attn_layer_fwd) and of a
Griffin stack (recurrent, recurrent, attention) against the CPU oracle.

Tolerances as for the recurrent residual layer: 1e-5 for fp32 and 3e-2 for
bf16 (the attention path's 2e-2 carried through the output projection and the
MLP, whose measured error gain is 1.4).  bf16 references compose the oracle's
functions with the interface's storage rounding at every stored tensor (the
normed inputs, q, k, v before and after the rotary embedding, the attention
output, x~, the MLP activations).  The full-size launch (2B width, 10 heads of
256, window 2048, d_ff = 3 d_model) is checked on a 96-token prefix of one
stream.
"""
import numpy as np
import pytest
import torch

import gated_linear_recurrence_02_amd as glr
import oracle
import synth
from problems import TOL, from_dev, make_problem, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL_LAYER_BF16 = 3e-2


def _say(*a):
    print(*a, flush=True)


def _cmp(name, got, ref, tol):
    err = oracle.rel_err(got, ref)
    _say(f"  {name}: err {err:.3e} (tol {tol:g})")
    assert np.all(np.isfinite(got)), f"{name} has non-finite values"
    assert err <= tol, f"{name}: {err} > {tol}"


def _setup(cfg, B, T, dm, Hq, dh, F, io):
    ap = synth.make_attn_proj(cfg, dm, Hq, dh, io)
    lp = synth.make_layer_params(cfg, dm, F, io)
    x = synth.make_activation(cfg, "block_x", (B, T, dm), io)
    return ap, lp, x


def _dev(ap, lp):
    return (glr.AttnProjWeights(*(to_dev(a, DEV) for a in (ap.wq, ap.wk, ap.wv, ap.wo))),
            glr.LayerWeights(to_dev(lp.tnorm_w, DEV), to_dev(lp.cnorm_w, DEV), to_dev(lp.gate_w, DEV),
                             to_dev(lp.up_w, DEV), to_dev(lp.down_w, DEV)))


def _ref(ap, lp, x, Hq, W, scale, rot, pos0, io, stored):
    Wd = synth.widen
    x64 = Wd(x)
    if not stored:
        return oracle.attn_layer(x64, Wd(lp.tnorm_w), Wd(lp.cnorm_w), Wd(ap.wq), Wd(ap.wk), Wd(ap.wv), Wd(ap.wo),
                                 Wd(lp.gate_w), Wd(lp.up_w), Wd(lp.down_w), Hq=Hq, window=W, scale=scale, rot=rot,
                                 pos0=pos0)
    st = lambda a: synth.widen(synth.store(a, io))
    B, T, dm = x64.shape
    dh = ap.wk.shape[0]
    xn = st(oracle.rmsnorm(x64, Wd(lp.tnorm_w)))
    pos = pos0 + np.arange(T)[None, :].repeat(B, axis=0)
    q = st(oracle.rope(st(oracle.linear(xn, Wd(ap.wq))).reshape(B, T, Hq, dh), pos, rot))
    k = st(oracle.rope(st(oracle.linear(xn, Wd(ap.wk))).reshape(B, T, 1, dh), pos, rot)).reshape(B, T, dh)
    v = st(oracle.linear(xn, Wd(ap.wv)))
    o = st(oracle.attn_fwd(q, k, v, W, scale)).reshape(B, T, Hq * dh)
    xt = st(x64 + oracle.linear(o, Wd(ap.wo)))
    xn2 = st(oracle.rmsnorm(xt, Wd(lp.cnorm_w)))
    a = st(oracle.gelu_tanh(st(oracle.linear(xn2, Wd(lp.gate_w)))) * st(oracle.linear(xn2, Wd(lp.up_w))))
    return xt + oracle.linear(a, Wd(lp.down_w))


@pytest.mark.parametrize("T,W,rot,pos0", [(37, 9, 8, 5), (20, 64, 16, 0), (1, 4, 0, 3)])
def test_attn_layer_fp32(T, W, rot, pos0):
    B, dm, Hq, dh, F = 2, 48, 3, 16, 64
    ap, lp, x = _setup(0, B, T, dm, Hq, dh, F, "f32")
    _say(f"attention layer fp32: B={B} T={T} d_model={dm} Hq={Hq} dh={dh} W={W} rot={rot} pos0={pos0}")
    apd, lwd = _dev(ap, lp)
    kc = torch.zeros((B, W, dh), dtype=torch.float32, device=DEV)
    vc = torch.zeros_like(kc)
    y = glr.attn_layer_fwd(to_dev(x, DEV), apd, lwd, Hq, W, scale=0.25, rot=rot, pos0=pos0, kcache=kc, vcache=vc)
    torch.cuda.synchronize()
    _cmp("y", from_dev(y), _ref(ap, lp, x, Hq, W, 0.25, rot, pos0, "f32", False), TOL["f32"])
    # the ring holds the rotated keys of the last min(T, W) positions
    xn = oracle.rmsnorm(synth.widen(x), synth.widen(lp.tnorm_w))
    pos = pos0 + np.arange(T)[None, :].repeat(B, axis=0)
    kr = oracle.rope(oracle.linear(xn, synth.widen(ap.wk)).reshape(B, T, 1, dh), pos, rot).reshape(B, T, dh)
    got = from_dev(kc)
    for t in range(max(0, T - W), T):
        _cmp(f"ring slot of t={t}", got[:, t % W], kr[:, t], TOL["f32"])


def test_attn_layer_bf16_2b_width_short():
    B, T, dm, Hq, dh, F, W = 1, 80, 2560, 10, 256, 7680, 64
    ap, lp, x = _setup(1, B, T, dm, Hq, dh, F, "bf16")
    apd, lwd = _dev(ap, lp)
    y = from_dev(glr.attn_layer_fwd(to_dev(x, DEV), apd, lwd, Hq, W, scale=1 / 16, rot=128))
    ref = _ref(ap, lp, x, Hq, W, 1 / 16, 128, 0, "bf16", True)
    _say(f"  (y against the all-double layer: {oracle.rel_err(y, _ref(ap, lp, x, Hq, W, 1 / 16, 128, 0, 'bf16', False)):.3e})")
    _cmp("y", y, ref, TOL_LAYER_BF16)


def test_attn_layer_full_size_prefix():
    B, T, dm, Hq, dh, F, W = 8, 2048, 2560, 10, 256, 7680, 2048
    ap, lp, x = _setup(1, B, T, dm, Hq, dh, F, "bf16")
    _say(f"attention layer bf16 full size: B={B} T={T} Hq={Hq} dh={dh} W={W}; oracle on stream 5, 96 tokens")
    apd, lwd = _dev(ap, lp)
    y = from_dev(glr.attn_layer_fwd(to_dev(x, DEV), apd, lwd, Hq, W, scale=1 / 16, rot=128))
    ref = _ref(ap, lp, np.ascontiguousarray(x[5:6, :96]), Hq, W, 1 / 16, 128, 0, "bf16", True)
    _cmp("y[5, :96]", y[5:6, :96], ref, TOL_LAYER_BF16)


def test_griffin_stack_rec_rec_attn():
    # Griffin's 2:1 pattern on a small fp32 model: two recurrent layers, one
    # attention layer, each a library call, against the oracle composition
    B, T, dm, F = 2, 30, 64, 96
    Hq, dh, W = 4, 16, 8
    x = synth.make_activation(0, "block_x", (B, T, dm), "f32")
    y = to_dev(x, DEV)
    ref = synth.widen(x)
    Wd = synth.widen
    for li in range(2):
        prob = make_problem(0, B=B, T=1)
        bp = synth.make_block_params(50 + li, dm, prob.D, "f32")
        lp = synth.make_layer_params(60 + li, dm, F, "f32")
        bw = glr.BlockWeights(to_dev(bp.proj_in_1, DEV), to_dev(bp.proj_in_2, DEV), to_dev(bp.proj_out, DEV))
        lw = glr.LayerWeights(to_dev(lp.tnorm_w, DEV), to_dev(lp.cnorm_w, DEV), to_dev(lp.gate_w, DEV),
                              to_dev(lp.up_w, DEV), to_dev(lp.down_w, DEV))
        y, _, _ = glr.layer_fwd(y, prob.weights(DEV), bw, lw)
        ref, _, _ = oracle.hawk_layer(ref, Wd(lp.tnorm_w), Wd(lp.cnorm_w), Wd(bp.proj_in_1), Wd(bp.proj_in_2),
                                      Wd(bp.proj_out), **prob.oracle_params(), gate_w=Wd(lp.gate_w),
                                      up_w=Wd(lp.up_w), down_w=Wd(lp.down_w), c=8.0)
    ap, lp, _ = _setup(70, B, T, dm, Hq, dh, F, "f32")
    apd, lwd = _dev(ap, lp)
    y = glr.attn_layer_fwd(y, apd, lwd, Hq, W, scale=0.25, rot=dh)
    ref = oracle.attn_layer(ref, Wd(lp.tnorm_w), Wd(lp.cnorm_w), Wd(ap.wq), Wd(ap.wk), Wd(ap.wv), Wd(ap.wo),
                            Wd(lp.gate_w), Wd(lp.up_w), Wd(lp.down_w), Hq=Hq, window=W, scale=0.25, rot=dh)
    torch.cuda.synchronize()
    _cmp("griffin stack y", from_dev(y), ref, TOL["f32"])
