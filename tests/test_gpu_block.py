"""GPU parity of the recurrent block (rglru_block_fwd) against the CPU oracle.

The block: out = proj_out(RG-LRU(conv(proj_in_1 x)) * GeLU(proj_in_2 x)) (page
"Griffin Guide: RecurrentGemma, RG-LRU & Hybrid Attention", "The Recurrent
Block Architecture", and the listing's RecurrentBlock).  Same metric and
tolerances as the scan: max |g - o| / max(|o|, RMS(o)) per output, 1e-5 for
fp32 I/O, 2e-2 for bf16 I/O.  The oracle keeps every intermediate in double.
The block's interface stores b1, b2 and the merged product in the I/O type;
for bf16 the reference composes the oracle's functions with that same
storage rounding at those three points (the rounding of synth/, which is the
input recipe's), so that the 2e-2 bar measures the path rather than three
extra bf16 roundings; the error against the all-double composition is
printed beside it.  The full-size case runs the 2B-width prefill shape
(B=8, T=2048, D = d_model = 2560) and checks one whole stream: the block is
causal and streams are independent, so a stream is a problem of its own.
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


def _say(*a):
    print(*a, flush=True)


def _cmp(name, got, ref, tol):
    err = oracle.rel_err(got, ref)
    _say(f"  {name}: err {err:.3e} (tol {tol:g})")
    assert np.all(np.isfinite(got)), f"{name} has non-finite values"
    assert err <= tol, f"{name}: {err} > {tol}"


def _block_setup(cfg, B, T, d_model, with_state):
    prob = make_problem(cfg, B=B, T=1, with_state=with_state)
    bp = synth.make_block_params(cfg, d_model, prob.D, prob.io)
    x = synth.make_activation(cfg, "block_x", (B, T, d_model), prob.io)
    return prob, bp, x


def _dev_block(bp):
    return glr.BlockWeights(to_dev(bp.proj_in_1, DEV), to_dev(bp.proj_in_2, DEV), to_dev(bp.proj_out, DEV))


def _oracle_block(prob, bp, x, b0, b1, T=None, with_state=False):
    xs = synth.widen(x[b0:b1, :T])
    h0 = prob.h0[b0:b1].astype(np.float64) if with_state else None
    hist = synth.widen(prob.hist[b0:b1]) if with_state else None
    return oracle.block_fwd(xs, synth.widen(bp.proj_in_1), synth.widen(bp.proj_in_2),
                            synth.widen(bp.proj_out), **prob.oracle_params(), h0=h0, hist_in=hist,
                            c=8.0)


def _oracle_block_stored(prob, bp, x, b0, b1, with_state=False):
    """The block with b1, b2 and the merged product stored in the I/O type."""
    def st(a):
        return synth.widen(synth.store(a, prob.io))
    xs = synth.widen(x[b0:b1])
    h0 = prob.h0[b0:b1].astype(np.float64) if with_state else None
    hist = synth.widen(prob.hist[b0:b1]) if with_state else None
    br1 = st(oracle.linear(xs, synth.widen(bp.proj_in_1)))
    br2 = st(oracle.linear(xs, synth.widen(bp.proj_in_2)))
    y, h_last, hist_out = oracle.fwd(br1, **prob.oracle_params(), h0=h0, hist_in=hist, c=8.0)
    out = oracle.linear(st(oracle.merge(y, br2)), synth.widen(bp.proj_out))
    return out, h_last, hist_out


def _run(prob, bp, x, with_state):
    w = prob.weights(DEV)
    h0 = to_dev(prob.h0, DEV) if with_state else None
    hist = to_dev(prob.hist, DEV) if with_state else None
    out, hl, ho = glr.block_fwd(to_dev(x, DEV), w, _dev_block(bp), h0=h0, hist_in=hist)
    torch.cuda.synchronize()
    return from_dev(out), from_dev(hl), from_dev(ho)


@pytest.mark.parametrize("T,d_model", [(100, 192), (32, 256), (7, 200)])
def test_block_fp32_small(T, d_model):
    # D = 256 (one gate block); d_model differs from D so that a transposed
    # projection would not even have the right shape; T ragged / one chunk / short
    prob, bp, x = _block_setup(0, 2, T, d_model, with_state=True)
    _say(f"block fp32: B=2 T={T} D={prob.D} d_model={d_model}, with state")
    out, hl, ho = _run(prob, bp, x, True)
    ro, rh, rhist = _oracle_block(prob, bp, x, 0, 2, with_state=True)
    _cmp("out", out, ro, TOL["f32"])
    _cmp("h_last", hl, rh, TOL["f32"])
    # hist_out holds the last 3 branch-1 activations, which are computed (proj_in_1 x)
    _cmp("hist_out", ho, rhist, TOL["f32"])


def test_block_bf16_2b_width_short():
    prob, bp, x = _block_setup(1, 2, 70, 2560, with_state=True)
    _say(f"block bf16: B=2 T=70 D={prob.D} H={prob.H} d_model=2560, with state")
    out, hl, ho = _run(prob, bp, x, True)
    ro, rh, rhist = _oracle_block_stored(prob, bp, x, 0, 2, with_state=True)
    _say(f"  (out against the all-double block: {oracle.rel_err(out, _oracle_block(prob, bp, x, 0, 2, with_state=True)[0]):.3e})")
    _cmp("out", out, ro, TOL["bf16"])
    _cmp("h_last", hl, rh, TOL["bf16"])
    # hist_out holds branch-1 activations, which the library rounds to bf16
    _cmp("hist_out", ho, rhist, TOL["bf16"])


@pytest.mark.parametrize("T,d_model", [(70, 200), (33, 320)])
def test_block_bf16_ragged_projection_shapes(T, d_model):
    # the projections' edge cases on the matrix-core GEMM and its fallback:
    # d_model = 200 sends proj_in (inner size 200) to the generic kernel and
    # gives proj_out a partial 256-column tile; d_model = 320 runs proj_in on
    # the matrix cores (inner size 5 x 64) and proj_out over a full and a
    # partial column tile; B T = 140 / 66 rows are one partial row tile
    prob, bp, x = _block_setup(1, 2, T, d_model, with_state=True)
    _say(f"block bf16: B=2 T={T} D={prob.D} d_model={d_model}, with state")
    out, hl, ho = _run(prob, bp, x, True)
    ro, rh, rhist = _oracle_block_stored(prob, bp, x, 0, 2, with_state=True)
    _cmp("out", out, ro, TOL["bf16"])
    _cmp("h_last", hl, rh, TOL["bf16"])
    _cmp("hist_out", ho, rhist, TOL["bf16"])


@pytest.mark.parametrize("T,d_model", [(33, 320), (300, 576)])
def test_block_gemm_tile_widths_agree(T, d_model, monkeypatch):
    # the projections' two matrix-core tile widths (256 and 128 output
    # columns) accumulate every output in the same order over K, so forced
    # either way (partial row and column tiles included) the block gives the
    # same bits, and the oracle's values
    prob, bp, x = _block_setup(1, 2, T, d_model, with_state=True)
    runs = {}
    for width in ("256", "128"):
        monkeypatch.setenv("RGLRU_GEMM_TILE_N", width)
        _say(f"block bf16: B=2 T={T} d_model={d_model}, GEMM tiles {width} wide")
        runs[width] = _run(prob, bp, x, True)
    monkeypatch.delenv("RGLRU_GEMM_TILE_N")
    for k, name in enumerate(("out", "h_last", "hist_out")):
        assert np.array_equal(runs["256"][k], runs["128"][k]), f"{name} depends on the GEMM tile width"
    ro, rh, _ = _oracle_block_stored(prob, bp, x, 0, 2, with_state=True)
    _cmp("out", runs["256"][0], ro, TOL["bf16"])
    _cmp("h_last", runs["256"][1], rh, TOL["bf16"])


def test_block_prefill_split_equals_whole():
    # two calls that hand over (h_last, hist_out) equal one call over the whole
    # sequence, and both equal the oracle
    prob, bp, x = _block_setup(0, 1, 90, 128, with_state=False)
    w = prob.weights(DEV)
    bw = _dev_block(bp)
    xd = to_dev(x, DEV)
    o1, h1, s1 = glr.block_fwd(xd[:, :50].contiguous(), w, bw)
    o2, h2, _ = glr.block_fwd(xd[:, 50:].contiguous(), w, bw, h0=h1, hist_in=s1)
    torch.cuda.synchronize()
    ro, rh, _ = _oracle_block(prob, bp, x, 0, 1)
    _cmp("split out", np.concatenate([from_dev(o1), from_dev(o2)], axis=1), ro, TOL["f32"])
    _cmp("split h_last", from_dev(h2), rh, TOL["f32"])


def test_block_full_size_one_stream():
    B, T, dm = 8, 2048, 2560
    prob, bp, x = _block_setup(1, B, T, dm, with_state=False)
    _say(f"block bf16 full size: B={B} T={T} D={prob.D} d_model={dm}; oracle on stream 5")
    out, hl, _ = _run(prob, bp, x, False)
    ro, rh, _ = _oracle_block_stored(prob, bp, x, 5, 6)
    _say(f"  (out[5] against the all-double block: {oracle.rel_err(out[5:6], _oracle_block(prob, bp, x, 5, 6)[0]):.3e})")
    _cmp("out[5]", out[5:6], ro, TOL["bf16"])
    _cmp("h_last[5]", hl[5:6], rh, TOL["bf16"])


@pytest.mark.parametrize("swap", [False, True])
def test_block_projection_weights_in_one_buffer(swap):
    # the two input projections as views of one allocation, in either order:
    # each projection reads its own weight, wherever it sits
    prob, bp, x = _block_setup(0, 1, 45, 160, with_state=False)
    w = prob.weights(DEV)
    both = torch.empty((2,) + bp.proj_in_1.shape, dtype=torch.float32, device=DEV)
    i1, i2 = (1, 0) if swap else (0, 1)
    both[i1] = to_dev(bp.proj_in_1, DEV)
    both[i2] = to_dev(bp.proj_in_2, DEV)
    bw = glr.BlockWeights(both[i1], both[i2], to_dev(bp.proj_out, DEV))
    out, hl, _ = glr.block_fwd(to_dev(x, DEV), w, bw)
    torch.cuda.synchronize()
    ro, rh, _ = _oracle_block(prob, bp, x, 0, 1)
    _cmp(f"out (swap={swap})", from_dev(out), ro, TOL["f32"])
    _cmp(f"h_last (swap={swap})", from_dev(hl), rh, TOL["f32"])


def test_block_single_token_with_state():
    # T = 1: the conv reads only the history; one chunk of one token
    prob, bp, x = _block_setup(0, 3, 1, 64, with_state=True)
    out, hl, ho = _run(prob, bp, x, True)
    ro, rh, rhist = _oracle_block(prob, bp, x, 0, 3, with_state=True)
    _cmp("out", out, ro, TOL["f32"])
    _cmp("h_last", hl, rh, TOL["f32"])
    _cmp("hist_out", ho, rhist, TOL["f32"])
