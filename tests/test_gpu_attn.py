"""GPU parity of the local sliding-window MQA (rglru_attn_fwd, rglru_attn_step)
against the CPU oracle.

Same metric as the scan: max |g - o| / max(|o|, RMS(o)) per output, 1e-5 for
fp32 I/O (vector-ALU path), 2e-2 for bf16 I/O (matrix-core path for dh = 256,
probabilities rounded to bf16 for the P V product).  Full-size shapes (the
2B-width prefill as 10 query heads of 256, the 32k-token prefill, 256 decode
streams with a 2048-slot ring) are checked on sampled tokens: the oracle's
decode step over a ring filled with the token's window gives exactly that
token's prefill output (a pin of the oracle), at a cost of one window per
token.
"""
import numpy as np
import pytest
import torch

import gated_linear_recurrence_02_amd as glr
import oracle
import synth
from problems import TOL, from_dev, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CFG = 20   # seed namespace of the attention inputs


def _say(*a):
    print(*a, flush=True)


def _cmp(name, got, ref, tol):
    err = oracle.rel_err(got, ref)
    _say(f"  {name}: err {err:.3e} (tol {tol:g})")
    assert np.all(np.isfinite(got)), f"{name} has non-finite values"
    assert err <= tol, f"{name}: {err} > {tol}"


def _qkv(B, T, Hq, dh, io, tag=0):
    q = synth.make_activation(CFG + tag, "attn_q", (B, T, Hq, dh), io)
    k = synth.make_activation(CFG + tag, "attn_k", (B, T, dh), io)
    v = synth.make_activation(CFG + tag, "attn_v", (B, T, dh), io)
    return q, k, v


def _oracle_token(q, k, v, b, t, W, scale):
    """The prefill output of token t of stream b, through the oracle's decode
    step over a ring that holds the token's window."""
    dh = k.shape[-1]
    lo = max(0, t - W + 1)
    kc = np.zeros((1, W, dh))
    vc = np.zeros((1, W, dh))
    for p in range(lo, t):
        kc[0, p % W] = synth.widen(k[b, p])
        vc[0, p % W] = synth.widen(v[b, p])
    return oracle.attn_step(synth.widen(q[b:b + 1, t]), synth.widen(k[b:b + 1, t]), synth.widen(v[b:b + 1, t]),
                            kc, vc, np.array([t]), scale)[0]


@pytest.mark.parametrize("B,T,Hq,dh,W", [(1, 256, 1, 256, 64), (2, 100, 3, 64, 17), (1, 40, 2, 8, 1)])
def test_prefill_fp32(B, T, Hq, dh, W):
    q, k, v = _qkv(B, T, Hq, dh, "f32")
    sc = dh ** -0.5
    _say(f"attn prefill fp32 B={B} T={T} Hq={Hq} dh={dh} W={W}")
    o = glr.attn_fwd(to_dev(q, DEV), to_dev(k, DEV), to_dev(v, DEV), W, sc)
    torch.cuda.synchronize()
    _cmp("o", from_dev(o), oracle.attn_fwd(synth.widen(q), synth.widen(k), synth.widen(v), W, sc), TOL["f32"])


@pytest.mark.parametrize("B,T,Hq,W", [(2, 200, 10, 64), (1, 300, 10, 2048), (2, 77, 1, 33), (1, 150, 16, 1),
                                      (1, 64, 5, 32)])
def test_prefill_bf16_mfma(B, T, Hq, W):
    # ragged against the 128-row workgroups and the 32-key tiles; W > T; W = 1
    q, k, v = _qkv(B, T, Hq, 256, "bf16")
    sc = 1.0 / 16
    _say(f"attn prefill bf16 B={B} T={T} Hq={Hq} dh=256 W={W}")
    o = glr.attn_fwd(to_dev(q, DEV), to_dev(k, DEV), to_dev(v, DEV), W, sc)
    torch.cuda.synchronize()
    _cmp("o", from_dev(o), oracle.attn_fwd(synth.widen(q), synth.widen(k), synth.widen(v), W, sc), TOL["bf16"])


def test_prefill_bf16_generic_shape():
    # bf16 with dh != 256 takes the vector-ALU path
    q, k, v = _qkv(1, 90, 4, 128, "bf16")
    o = glr.attn_fwd(to_dev(q, DEV), to_dev(k, DEV), to_dev(v, DEV), 20, 0.1)
    torch.cuda.synchronize()
    _cmp("o", from_dev(o), oracle.attn_fwd(synth.widen(q), synth.widen(k), synth.widen(v), 20, 0.1), TOL["bf16"])


@pytest.mark.parametrize("B,T,W,tokens", [(8, 2048, 2048, [(0, 0), (3, 31), (7, 1000), (5, 2047)]),
                                          (1, 32768, 2048, [(0, 2047), (0, 2048), (0, 20000), (0, 32767)])])
def test_prefill_full_size_sampled(B, T, W, tokens):
    Hq, dh = 10, 256
    q, k, v = _qkv(B, T, Hq, dh, "bf16", tag=1)
    _say(f"attn prefill full size B={B} T={T} Hq={Hq} dh={dh} W={W}; tokens {tokens}")
    o = from_dev(glr.attn_fwd(to_dev(q, DEV), to_dev(k, DEV), to_dev(v, DEV), W, 1.0 / 16))
    for b, t in tokens:
        _cmp(f"o[{b},{t}]", o[b, t], _oracle_token(q, k, v, b, t, W, 1.0 / 16), TOL["bf16"])


def _decode_run(B, Hq, dh, W, io, starts, steps, tag):
    """Streams b begin at position starts[b] with their earlier window already
    in the ring; both sides run `steps` decode steps."""
    rng_q = synth.make_activation(CFG + tag, "attn_q", (steps, B, Hq, dh), io)
    rng_k = synth.make_activation(CFG + tag, "attn_k", (steps, B, dh), io)
    rng_v = synth.make_activation(CFG + tag, "attn_v", (steps, B, dh), io)
    hist_k = synth.make_activation(CFG + tag, "attn_hk", (B, W, dh), io)
    hist_v = synth.make_activation(CFG + tag, "attn_hv", (B, W, dh), io)
    kc, vc = to_dev(hist_k, DEV), to_dev(hist_v, DEV)
    okc, ovc = synth.widen(hist_k), synth.widen(hist_v)
    pos = torch.tensor(starts, dtype=torch.int32, device=DEV)
    sc = dh ** -0.5
    worst = 0.0
    for s in range(steps):
        o = glr.attn_step(to_dev(rng_q[s], DEV), to_dev(rng_k[s], DEV), to_dev(rng_v[s], DEV), kc, vc, pos, sc)
        ref = oracle.attn_step(synth.widen(rng_q[s]), synth.widen(rng_k[s]), synth.widen(rng_v[s]), okc, ovc,
                               np.array(starts) + s, sc)
        worst = max(worst, oracle.rel_err(from_dev(o), ref))
        pos += 1
    torch.cuda.synchronize()
    return worst, kc, vc, okc, ovc


@pytest.mark.parametrize("io,dh,Hq", [("bf16", 256, 10), ("bf16", 256, 16), ("f32", 64, 3), ("bf16", 128, 4)])
def test_decode_ring_wraps(io, dh, Hq):
    # different start positions per stream, from a fresh stream (0) to one deep
    # past the window; the ring wraps during the run
    B, W, steps = 4, 40, 60
    starts = [0, 7, 39, 500]
    _say(f"attn decode {io} dh={dh} Hq={Hq} W={W} starts {starts} steps {steps}")
    worst, kc, vc, okc, ovc = _decode_run(B, Hq, dh, W, io, starts, steps, tag=2)
    _say(f"  worst step err {worst:.3e}")
    assert worst <= TOL[io]
    # the rings match slot for slot (positions written by the steps are copies)
    assert np.array_equal(from_dev(kc), okc) and np.array_equal(from_dev(vc), ovc)


def test_decode_fresh_cache_never_reads_unwritten_slots():
    # a ring full of NaN: the first W steps from position 0 must not see it
    B, Hq, dh, W = 2, 10, 256, 64
    kc = torch.full((B, W, dh), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full((B, W, dh), float("nan"), dtype=torch.bfloat16, device=DEV)
    q, k, v = _qkv(B, 70, Hq, dh, "bf16", tag=3)
    ref = oracle.attn_fwd(synth.widen(q), synth.widen(k), synth.widen(v), W, 1.0 / 16)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    qd, kd, vd = to_dev(q, DEV), to_dev(k, DEV), to_dev(v, DEV)
    worst = 0.0
    for t in range(70):
        o = glr.attn_step(qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(), kc, vc, pos, 1.0 / 16)
        worst = max(worst, oracle.rel_err(from_dev(o), ref[:, t]))
        pos += 1
    torch.cuda.synchronize()
    _say(f"  fresh-cache decode vs prefill oracle: worst {worst:.3e}")
    assert worst <= TOL["bf16"]


def test_prefill_then_decode():
    # the prefill fills the ring; decode continues at pos = T; together they
    # equal the oracle's prefill over the whole sequence
    B, T0, T1, Hq, dh, W = 2, 150, 30, 10, 256, 64
    q, k, v = _qkv(B, T0 + T1, Hq, dh, "bf16", tag=4)
    ref = oracle.attn_fwd(synth.widen(q), synth.widen(k), synth.widen(v), W, 1.0 / 16)
    qd, kd, vd = to_dev(q, DEV), to_dev(k, DEV), to_dev(v, DEV)
    kc = torch.empty((B, W, dh), dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    o0 = glr.attn_fwd(qd[:, :T0].contiguous(), kd[:, :T0].contiguous(), vd[:, :T0].contiguous(), W, 1.0 / 16,
                      kcache=kc, vcache=vc)
    pos = torch.full((B,), T0, dtype=torch.int32, device=DEV)
    outs = []
    for t in range(T0, T0 + T1):
        outs.append(glr.attn_step(qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(), kc, vc,
                                  pos, 1.0 / 16))
        pos += 1
    torch.cuda.synchronize()
    _cmp("prefill part", from_dev(o0), ref[:, :T0], TOL["bf16"])
    _cmp("decode part", np.stack([from_dev(x) for x in outs], axis=1), ref[:, T0:], TOL["bf16"])


def test_decode_full_size_sampled():
    # 256 streams, ring of 2048 slots, every stream deep past the window
    B, Hq, dh, W = 256, 10, 256, 2048
    hk = synth.make_activation(CFG + 5, "attn_hk", (B, W, dh), "bf16")
    hv = synth.make_activation(CFG + 5, "attn_hv", (B, W, dh), "bf16")
    qt = synth.make_activation(CFG + 5, "attn_q", (B, Hq, dh), "bf16")
    kt = synth.make_activation(CFG + 5, "attn_k", (B, dh), "bf16")
    vt = synth.make_activation(CFG + 5, "attn_v", (B, dh), "bf16")
    starts = np.array([4096 + 13 * b for b in range(B)])
    kc, vc = to_dev(hk, DEV), to_dev(hv, DEV)
    pos = torch.tensor(starts, dtype=torch.int32, device=DEV)
    o = from_dev(glr.attn_step(to_dev(qt, DEV), to_dev(kt, DEV), to_dev(vt, DEV), kc, vc, pos, 1.0 / 16))
    for b in (0, 77, 255):
        okc, ovc = synth.widen(hk[b:b + 1]), synth.widen(hv[b:b + 1])
        ref = oracle.attn_step(synth.widen(qt[b:b + 1]), synth.widen(kt[b:b + 1]), synth.widen(vt[b:b + 1]),
                               okc, ovc, starts[b:b + 1], 1.0 / 16)
        _cmp(f"o_t[{b}]", o[b:b + 1], ref, TOL["bf16"])
        assert np.array_equal(from_dev(kc[b:b + 1]), okc)


@pytest.mark.parametrize("io,dh", [("bf16", 256), ("f32", 32)])
def test_prefill_single_token_and_ring_fill(io, dh):
    # T = 1 and T < W: o equals v for the lone token; the ring receives it in slot 0
    B, Hq, W = 3, 4, 16
    q, k, v = _qkv(B, 1, Hq, dh, io, tag=6)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    kc = torch.zeros((B, W, dh), dtype=dt, device=DEV)
    vc = torch.zeros_like(kc)
    o = glr.attn_fwd(to_dev(q, DEV), to_dev(k, DEV), to_dev(v, DEV), W, dh ** -0.5, kcache=kc, vcache=vc)
    torch.cuda.synchronize()
    _cmp("o", from_dev(o), np.repeat(synth.widen(v)[:, :, None, :], Hq, axis=2), TOL[io])
    assert np.array_equal(from_dev(kc[:, 0]), synth.widen(k[:, 0]))
    assert np.all(from_dev(kc[:, 1:]) == 0.0)
