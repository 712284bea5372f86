"""GPU parity of the forward entry points against the CPU oracle.

Metric: max |g - o| / max(|o|, RMS(o)) per output tensor; pass at 1e-5 for
fp32 I/O and 2e-2 for bf16 I/O with fp32 state.  Copies (conv history) must
match bit for bit.  Full-size workloads run in the launch configuration the
bench times and are checked on whole (stream, 256-channel block) slices,
each of which the oracle computes as a problem of its own (B = 1, D = 256,
H = 1): block-diagonal gates and channel-local conv/scan make such a slice
independent of every other.
"""
import numpy as np
import pytest
import torch

import gated_linear_recurrence_02_amd as glr
import oracle
import synth
from problems import TOL, Problem, from_dev, make_problem, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def _cmp(name, got, ref, tol):
    err = oracle.rel_err(got, ref)
    _say(f"  {name}: err {err:.3e} (tol {tol:g})")
    assert np.all(np.isfinite(got)), f"{name} has non-finite values"
    assert err <= tol, f"{name}: {err} > {tol}"


def _run_fwd(prob, mode="A", h0=None, hist=None):
    w = prob.weights(DEV)
    u = to_dev(prob.u, DEV)
    h0_d = None if h0 is None else to_dev(h0, DEV)
    hist_d = None if hist is None else to_dev(hist, DEV)
    if mode == "A":
        y, hl, ho = glr.scan_fwd(u, w, h0=h0_d, hist_in=hist_d)
    else:
        x, _ = glr.conv1d(u, w.conv_w, w.conv_b, hist_d, H=prob.H)
        y, hl, ho = glr.scan_fwd(x, w, h0=h0_d, conv=False)
    torch.cuda.synchronize()
    return y, hl, ho


def _oracle_slice(prob, b, h, h0=None, hist=None):
    u = synth.widen(prob.slice_block(prob.u, b, h))
    h0s = None if h0 is None else prob.slice_block(h0.astype(np.float64), b, h)
    hs = None if hist is None else synth.widen(prob.slice_block(hist, b, h))
    return oracle.fwd(u, **prob.oracle_params(h), h0=h0s, hist_in=hs)


# --------------------------------------------------------------- config 0
def test_config0_fp32_mode_a_full():
    prob = make_problem(0)
    _say("config 0: B=1 T=256 D=256 fp32, mode A")
    y, hl, _ = _run_fwd(prob)
    ry, rh, _ = oracle.fwd(synth.widen(prob.u), **prob.oracle_params())
    _cmp("y", from_dev(y), ry, TOL["f32"])
    _cmp("h_last", from_dev(hl), rh, TOL["f32"])


def test_config0_fp32_conv_gates_scan_stages():
    prob = make_problem(0, with_state=True)
    _say("config 0 stages: conv1d, gates, scan mode C, fp32")
    w = prob.weights(DEV)
    u = to_dev(prob.u, DEV)
    x, ho = glr.conv1d(u, w.conv_w, w.conv_b, to_dev(prob.hist, DEV))
    r, i = glr.gates(x, w)
    y, hl, _ = glr.scan_fwd(x, w, r=r, i=i, h0=to_dev(prob.h0, DEV))
    torch.cuda.synchronize()
    op = prob.oracle_params()
    rx, rho = oracle.conv1d(synth.widen(prob.u), op["conv_w"], op["conv_b"], synth.widen(prob.hist))
    _cmp("x", from_dev(x), rx, TOL["f32"])
    assert np.array_equal(ho.cpu().numpy(), prob.hist[:, :, :] if prob.T < 3 else prob.u[:, -3:, :])
    rr, ri = oracle.gates(from_dev(x), op["W_a"], op["b_a"], op["W_x"], op["b_x"])
    _cmp("r", from_dev(r), rr, TOL["f32"])
    _cmp("i", from_dev(i), ri, TOL["f32"])
    ry, rh = oracle.scan(from_dev(x), from_dev(r), from_dev(i), op["Lambda"], prob.h0.astype(np.float64))
    _cmp("y", from_dev(y), ry, TOL["f32"])
    _cmp("h_last", from_dev(hl), rh, TOL["f32"])


@pytest.mark.parametrize("B,T", [(2, 77), (8, 2048)])
def test_conv1d_bf16_against_oracle(B, T):
    # bf16 conv on the 2B-width taps, with a carried history: T = 77 ends in a
    # partial 32-token segment; the full prefill shape is checked on two
    # streams (the conv is per stream and per channel).  The only error is the
    # rounding of x to bf16; the history copy is bit for bit.
    prob = make_problem(1, B=B, T=T, with_state=True)
    _say(f"conv1d bf16: B={B} T={T} D=2560, history given")
    w = prob.weights(DEV)
    x, ho = glr.conv1d(to_dev(prob.u, DEV), w.conv_w, w.conv_b, to_dev(prob.hist, DEV), H=prob.H)
    torch.cuda.synchronize()
    op = prob.oracle_params()
    xs = from_dev(x)
    for b in sorted({0, B - 1}):
        rx, _ = oracle.conv1d(synth.widen(prob.u[b:b + 1]), op["conv_w"], op["conv_b"],
                              synth.widen(prob.hist[b:b + 1]))
        _cmp(f"x[b={b}]", xs[b:b + 1], rx, TOL["bf16"])
    want = np.concatenate([prob.hist, prob.u], axis=1)[:, -3:, :]
    assert np.array_equal(ho.cpu().view(torch.int16).numpy().view(np.uint16), want)


@pytest.mark.parametrize("B,T", [(2, 77), (8, 2048)])
def test_gates_bf16_blocks_and_ragged_rows(B, T):
    # the bf16 gate kernel on the 2B-width parameters; B*T = 2*77 rows is not a
    # multiple of the 32-row tile, and the conv output is the gate input; the
    # full prefill shape runs the persistent launch the bench times
    prob = make_problem(1, B=B, T=T)
    _say(f"gates: B={B} T={T} D=2560 bf16")
    w = prob.weights(DEV)
    x, _ = glr.conv1d(to_dev(prob.u, DEV), w.conv_w, w.conv_b, H=prob.H)
    r, i = glr.gates(x, w)
    torch.cuda.synchronize()
    xs = from_dev(x)
    for h in (0, 9):
        op = prob.oracle_params(h)
        rr, ri = oracle.gates(prob.slice_block(xs, None, h), op["W_a"], op["b_a"], op["W_x"], op["b_x"])
        _cmp(f"r[h={h}]", prob.slice_block(from_dev(r), None, h), rr, TOL["bf16"])
        _cmp(f"i[h={h}]", prob.slice_block(from_dev(i), None, h), ri, TOL["bf16"])


# ------------------------------------------------------ ragged / edge shapes
@pytest.mark.parametrize("T", [1, 2, 3, 17, 31, 32, 33, 95, 130])
def test_mode_a_ragged_lengths_with_state(T):
    prob = make_problem(1, B=2, T=T, with_state=True)
    _say(f"ragged T={T}, B=2, D=2560 bf16, h0 and history given")
    y, hl, ho = _run_fwd(prob, h0=prob.h0, hist=prob.hist)
    for b, h in [(0, 0), (1, 9), (1, 4)]:
        ry, rh, rho = _oracle_slice(prob, b, h, prob.h0, prob.hist)
        _cmp(f"y[b={b},h={h}]", prob.slice_block(from_dev(y), b, h), ry, TOL["bf16"])
        _cmp(f"h_last[b={b},h={h}]", prob.slice_block(from_dev(hl), b, h), rh, TOL["bf16"])
    want = np.concatenate([prob.hist, prob.u], axis=1)[:, -3:, :]
    assert np.array_equal(ho.cpu().view(torch.int16).numpy().view(np.uint16), want)


@pytest.mark.parametrize("B,T", [(48, 40), (130, 33)])
def test_mode_a_many_short_streams_with_state(B, T):
    # many streams, two chunks each (the second ragged): the claims run
    # through every stream's first chunk (unstaged, history-fed) before any
    # second chunk, whose look-back then finds its one predecessor
    prob = make_problem(1, B=B, T=T, with_state=True)
    _say(f"B={B} T={T}, D=2560 bf16, h0 and history given")
    y, hl, ho = _run_fwd(prob, h0=prob.h0, hist=prob.hist)
    for b, h in [(0, 0), (B // 2, 5), (B - 1, 9)]:
        ry, rh, rho = _oracle_slice(prob, b, h, prob.h0, prob.hist)
        _cmp(f"y[b={b},h={h}]", prob.slice_block(from_dev(y), b, h), ry, TOL["bf16"])
        _cmp(f"h_last[b={b},h={h}]", prob.slice_block(from_dev(hl), b, h), rh, TOL["bf16"])
    want = np.concatenate([prob.hist, prob.u], axis=1)[:, -3:, :]
    assert np.array_equal(ho.cpu().view(torch.int16).numpy().view(np.uint16), want)


def test_mode_a_bf16_extreme_decay_constants():
    # Lambda far out on both sides: softplus(-Lambda) underflowing to zero
    # (a_t = 1, the state carried unchanged), a normal but tiny decay
    # constant, one at the edge of the float range, and a_t ~ 0 (h_t ~ i_t x_t)
    prob = make_problem(1, B=2, T=100, with_state=True)
    lam = prob.params.Lambda
    K = prob.D // prob.H
    for h, v in [(0, 120.0), (1, 60.0), (2, 88.5), (3, -20.0), (4, 30.0)]:
        lam[h * K:(h + 1) * K] = v
    _say("mode A bf16, B=2 T=100, Lambda blocks 120, 60, 88.5, -20, 30, with state")
    y, hl, _ = _run_fwd(prob, h0=prob.h0, hist=prob.hist)
    for b, h in [(0, 0), (1, 1), (0, 2), (1, 3), (0, 4), (1, 7)]:
        ry, rh, _ = _oracle_slice(prob, b, h, prob.h0, prob.hist)
        _cmp(f"y[b={b},h={h}]", prob.slice_block(from_dev(y), b, h), ry, TOL["bf16"])
        _cmp(f"h_last[b={b},h={h}]", prob.slice_block(from_dev(hl), b, h), rh, TOL["bf16"])


def test_mode_b_equals_conv_then_mode_b_oracle():
    prob = make_problem(1, B=2, T=200)
    _say("mode B: B=2 T=200 D=2560 bf16 (x = conv output from rglru_conv1d)")
    w = prob.weights(DEV)
    x, _ = glr.conv1d(to_dev(prob.u, DEV), w.conv_w, w.conv_b, H=prob.H)
    y, hl, _ = glr.scan_fwd(x, w, conv=False)
    torch.cuda.synchronize()
    xs = x.cpu().view(torch.int16).numpy().view(np.uint16)
    for b, h in [(0, 3), (1, 8)]:
        op = prob.oracle_params(h)
        op["conv_w"] = None
        ry, rh, _ = oracle.fwd(synth.widen(prob.slice_block(xs, b, h)), **op)
        _cmp(f"y[b={b},h={h}]", prob.slice_block(from_dev(y), b, h), ry, TOL["bf16"])
        _cmp(f"h_last[b={b},h={h}]", prob.slice_block(from_dev(hl), b, h), rh, TOL["bf16"])


def test_mode_c_scan_only_any_width():
    # scan stage only on a width that is not a multiple of 256
    B, T, D = 3, 77, 300
    rng_x = synth.make_activation(1, "u", (B, T, D), "bf16")
    r = synth.store(0.02 + 0.96 * synth.uniform(5, 0, B * T * D), "bf16").reshape(B, T, D)
    i = synth.store(0.02 + 0.96 * synth.uniform(6, 0, B * T * D), "bf16").reshape(B, T, D)
    lam = synth.make_params(1, D, 1, "bf16").Lambda
    h0 = synth.store(synth.normal(7, 0, B * D), "f32").reshape(B, D)
    _say(f"mode C: B={B} T={T} D={D} bf16")
    w = glr.Weights(conv_w=None, W_a=None, W_x=None, Lambda=to_dev(lam, DEV))
    y, hl, _ = glr.scan_fwd(to_dev(rng_x, DEV), w, r=to_dev(r, DEV), i=to_dev(i, DEV),
                            h0=to_dev(h0, DEV))
    torch.cuda.synchronize()
    ry, rh = oracle.scan(synth.widen(rng_x), synth.widen(r), synth.widen(i), synth.widen(lam),
                         h0.astype(np.float64))
    _cmp("y", from_dev(y), ry, TOL["bf16"])
    _cmp("h_last", from_dev(hl), rh, TOL["bf16"])


# ---------------------------------------------------- full-size workloads
def test_config1_full_size_every_block():
    # every 256-channel block on one stream (stream h % B), the first and the
    # last block also on the other ends of the batch
    prob = make_problem(1)
    _say("config 1 full size: B=8 T=2048 D=2560 bf16, mode A")
    y, hl, _ = _run_fwd(prob)
    yn, hn = from_dev(y), from_dev(hl)
    assert np.all(np.isfinite(yn))
    for b, h in [(h % prob.B, h) for h in range(prob.H)] + [(7, 0), (3, 9)]:
        ry, rh, _ = _oracle_slice(prob, b, h)
        _cmp(f"y[b={b},h={h}]", prob.slice_block(yn, b, h), ry, TOL["bf16"])
        _cmp(f"h_last[b={b},h={h}]", prob.slice_block(hn, b, h), rh, TOL["bf16"])
    glr.workspace_status(DEV)


def test_config2_full_size_every_block():
    prob = make_problem(2)
    _say("config 2 full size: B=1 T=32768 D=2560 bf16, mode A, every block")
    y, hl, _ = _run_fwd(prob)
    yn, hn = from_dev(y), from_dev(hl)
    assert np.all(np.isfinite(yn))
    for h in range(prob.H):
        ry, rh, _ = _oracle_slice(prob, 0, h)
        _cmp(f"y[h={h}]", prob.slice_block(yn, 0, h), ry, TOL["bf16"])
        _cmp(f"h_last[h={h}]", prob.slice_block(hn, 0, h), rh, TOL["bf16"])
    glr.workspace_status(DEV)


def test_config4_forward_full_size():
    # the 9B-width workload's forward (B=4 T=8192 D=4096 H=16): blocks 0, 8
    # and 15 over all streams, every other block on one stream
    prob = make_problem(4)
    _say("config 4 forward full size: B=4 T=8192 D=4096 H=16 bf16, mode A")
    y, hl, _ = _run_fwd(prob)
    yn, hn = from_dev(y), from_dev(hl)
    assert np.all(np.isfinite(yn))
    cases = [(b, h) for h in (0, 8, 15) for b in range(prob.B)]
    cases += [(h % prob.B, h) for h in range(prob.H) if h not in (0, 8, 15)]
    for b, h in cases:
        ry, rh, _ = _oracle_slice(prob, b, h)
        _cmp(f"y[b={b},h={h}]", prob.slice_block(yn, b, h), ry, TOL["bf16"])
        _cmp(f"h_last[b={b},h={h}]", prob.slice_block(hn, b, h), rh, TOL["bf16"])
    glr.workspace_status(DEV)


# ------------------------------------------------------- self-consistency
def test_split_equals_whole_on_gpu():
    prob = make_problem(1, B=2, T=150, with_state=True)
    w = prob.weights(DEV)
    u = to_dev(prob.u, DEV)
    h0 = to_dev(prob.h0, DEV)
    hist = to_dev(prob.hist, DEV)
    y, hl, ho = glr.scan_fwd(u, w, h0=h0, hist_in=hist)
    y1, hl1, ho1 = glr.scan_fwd(u[:, :67].contiguous(), w, h0=h0, hist_in=hist)
    y2, hl2, ho2 = glr.scan_fwd(u[:, 67:].contiguous(), w, h0=hl1, hist_in=ho1)
    torch.cuda.synchronize()
    yy = torch.cat([y1, y2], 1)
    _cmp("split y", from_dev(yy), from_dev(y), 1e-2)
    _cmp("split h_last", from_dev(hl2), from_dev(hl), 1e-4)
    assert torch.equal(ho2, ho)


def test_repeatable():
    # every entry point is bitwise repeatable, the chunked scan included: a
    # chunk folds the aggregates after the newest published end state onto it
    # in chunk order, which is the serial recurrence whatever the timing
    prob = make_problem(1, B=2, T=500)
    w = prob.weights(DEV)
    u = to_dev(prob.u, DEV)
    x1, _ = glr.conv1d(u, w.conv_w, w.conv_b, H=prob.H)
    x2, _ = glr.conv1d(u, w.conv_w, w.conv_b, H=prob.H)
    r1, i1 = glr.gates(x1, w)
    r2, i2 = glr.gates(x2, w)
    y1, h1, _ = glr.scan_fwd(u, w)
    y1, h1 = y1.clone(), h1.clone()
    assert torch.equal(x1, x2) and torch.equal(r1, r2) and torch.equal(i1, i2)
    for k in range(5):
        y2, h2, _ = glr.scan_fwd(u, w)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(h1, h2), f"scan differs on repeat {k}"
    # the long prefill, where a chunk looks back over many in-flight chunks
    prob2 = make_problem(2, T=8192)
    u2, w2 = to_dev(prob2.u, DEV), prob2.weights(DEV)
    ya, ha, _ = glr.scan_fwd(u2, w2)
    ya, ha = ya.clone(), ha.clone()
    for k in range(3):
        yb, hb, _ = glr.scan_fwd(u2, w2)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb) and torch.equal(ha, hb), f"long scan differs on repeat {k}"
    glr.workspace_status(DEV)


@pytest.mark.parametrize("mode", ["A", "C"])
def test_results_independent_of_grid(mode, monkeypatch):
    # the persistent forward claims its units at run time; one workgroup per
    # 256-channel group (every wait then on the same workgroup's earlier
    # units) and three must give the same bits as the full grid.  In mode A
    # the full grid here (25 workgroups per group, 4 streams) runs without the
    # look-back prefetch and the capped grids with it, so this also compares
    # the two look-back paths bit for bit
    prob = make_problem(1, B=4, T=700, with_state=True)
    w = prob.weights(DEV)
    u = to_dev(prob.u, DEV)
    h0, hist = to_dev(prob.h0, DEV), to_dev(prob.hist, DEV)
    if mode == "C":
        x, _ = glr.conv1d(u, w.conv_w, w.conv_b, hist, H=prob.H)
        r, i = glr.gates(x, w)
        wc = glr.Weights(conv_w=None, W_a=None, W_x=None, Lambda=w.Lambda)
        run = lambda: glr.scan_fwd(x, wc, r=r, i=i, h0=h0)
    else:
        run = lambda: glr.scan_fwd(u, w, h0=h0, hist_in=hist)
    y0, h0_, _ = run()
    y0, h0_ = y0.clone(), h0_.clone()
    for cap in ("1", "3"):
        monkeypatch.setenv("RGLRU_FWD_GROUP_WORKGROUPS", cap)
        _say(f"mode {mode}, B=4 T=700 D=2560, {cap} workgroup(s) per group")
        y1, h1, _ = run()
        torch.cuda.synchronize()
        assert torch.equal(y0, y1) and torch.equal(h0_, h1), f"results depend on the grid ({cap})"
    monkeypatch.delenv("RGLRU_FWD_GROUP_WORKGROUPS")
    ry, rh, _ = _oracle_slice(prob, 3, 5, prob.h0, prob.hist)
    _cmp("y[b=3,h=5]", prob.slice_block(from_dev(y0), 3, 5), ry, TOL["bf16"])
    glr.workspace_status(DEV)


def test_workspace_reused_across_shapes():
    # one zeroed forward workspace serves calls of any shape one after another:
    # the claim counters sit at fixed offsets, carry words carry their call's tag
    for T in (40, 1000, 7, 333):
        prob = make_problem(1, B=1, T=T)
        y, hl, _ = _run_fwd(prob)
        ry, rh, _ = _oracle_slice(prob, 0, 2)
        _cmp(f"T={T} y", prob.slice_block(from_dev(y), 0, 2), ry, TOL["bf16"])
    # a narrow call, then a call with 65 blocks on the same buffer: block 64's
    # counter lies past the 64 counters a narrow layout would have reserved
    for D, H, T in ((256, 1, 300), (16640, 65, 130)):
        p = synth.make_params(1, D, H, "bf16")
        u = synth.make_activation(1, "u", (2, T, D), "bf16")
        prob = Problem(1, 2, T, D, H, "bf16", p, u, None, None)
        y, hl, _ = _run_fwd(prob)
        yn, hn = from_dev(y), from_dev(hl)
        assert np.all(np.isfinite(yn))
        for b, h in sorted({(0, 0), (1, H - 1), (0, H // 2)}):
            ry, rh, _ = _oracle_slice(prob, b, h)
            _cmp(f"D={D} y[b={b},h={h}]", prob.slice_block(yn, b, h), ry, TOL["bf16"])
            _cmp(f"D={D} h_last[b={b},h={h}]", prob.slice_block(hn, b, h), rh, TOL["bf16"])
    glr.workspace_status(DEV)
    hdr = glr._ws_cache[(torch.device(DEV), "fwd")][0][:16].cpu().numpy().view(np.uint32)
    assert hdr[0] == 0 and hdr[1] == 0 and hdr[3] == 0     # counters reset, no look-back timeout


# --------------------------------------- opt-in one-wave-per-SIMD kernel
def test_fused_opt_in_kernel(monkeypatch):
    # RGLRU_FWD_FUSED=1 sends mode A bf16 to the second, one-wave-per-SIMD
    # forward; it answers to the same oracle, at full size, on ragged lengths
    # with state, and gives the same bits for any grid
    monkeypatch.setenv("RGLRU_FWD_FUSED", "1")
    prob = make_problem(1)
    _say("fused kernel, config 1 full size: B=8 T=2048 D=2560 bf16")
    y, hl, _ = _run_fwd(prob)
    yn, hn = from_dev(y), from_dev(hl)
    for b, h in [(0, 0), (7, 9), (3, 4), (5, 6)]:
        ry, rh, _ = _oracle_slice(prob, b, h)
        _cmp(f"y[b={b},h={h}]", prob.slice_block(yn, b, h), ry, TOL["bf16"])
        _cmp(f"h_last[b={b},h={h}]", prob.slice_block(hn, b, h), rh, TOL["bf16"])
    for T in (1, 3, 33, 130):
        prob = make_problem(1, B=2, T=T, with_state=True)
        _say(f"fused kernel, ragged T={T}, B=2, h0 and history given")
        y, hl, ho = _run_fwd(prob, h0=prob.h0, hist=prob.hist)
        for b, h in [(0, 0), (1, 9)]:
            ry, rh, _ = _oracle_slice(prob, b, h, prob.h0, prob.hist)
            _cmp(f"y[b={b},h={h}]", prob.slice_block(from_dev(y), b, h), ry, TOL["bf16"])
            _cmp(f"h_last[b={b},h={h}]", prob.slice_block(from_dev(hl), b, h), rh, TOL["bf16"])
        want = np.concatenate([prob.hist, prob.u], axis=1)[:, -3:, :]
        assert np.array_equal(ho.cpu().view(torch.int16).numpy().view(np.uint16), want)
    prob = make_problem(1, B=4, T=700)
    y0, h0_, _ = _run_fwd(prob)
    y0, h0_ = y0.clone(), h0_.clone()
    monkeypatch.setenv("RGLRU_FWD_GROUP_WORKGROUPS", "1")
    y1, h1, _ = _run_fwd(prob)
    assert torch.equal(y0, y1) and torch.equal(h0_, h1), "fused results depend on the grid"
    glr.workspace_status(DEV)
