"""GPU parity of rglru_step (decode) against the oracle.

The decode workload is B = 256 streams, D = 2560, 512 consecutive one-token
calls with the fp32 state and the 3-token conv history carried between calls.
The oracle's prefill over the same 512 tokens is, by definition, the same
computation (its own step-vs-prefill consistency is pinned on the CPU), so
every y_t of sampled (stream, block) slices is compared with it, as are the
final state and history.
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


def _say(*a):
    print(*a, flush=True)


def _cmp(name, got, ref, tol):
    err = oracle.rel_err(got, ref)
    _say(f"  {name}: err {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= tol, f"{name}: {err} > {tol}"


def _decode_run(steps, B=None, sample_streams=(0, 1, 77, 255), sample_heads=(0, 9)):
    cfg = synth.DECODE_256
    B = cfg.B if B is None else B
    D, H = cfg.D, cfg.H
    params = synth.make_params(cfg.idx, D, H, cfg.io)
    w = glr.Weights(conv_w=to_dev(params.conv_w, DEV), W_a=to_dev(params.W_a, DEV),
                    W_x=to_dev(params.W_x, DEV), Lambda=to_dev(params.Lambda, DEV),
                    conv_b=to_dev(params.conv_b, DEV), b_a=to_dev(params.b_a, DEV),
                    b_x=to_dev(params.b_x, DEV))
    # two history buffers, alternated; the first step reads no history (zeros)
    hists = [torch.full((B, 3, D), 7.0, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    h = torch.zeros((B, D), dtype=torch.float32, device=DEV)
    us, ys = [], []
    for s in range(steps):
        u_s = synth.make_activation(cfg.idx, "u", (cfg.B, D), cfg.io, start=s * cfg.B * D)[:B]
        us.append(u_s)
        y, _ = glr.step(to_dev(u_s, DEV), w, h, None if s == 0 else hists[s % 2], hists[(s + 1) % 2])
        ys.append(y)
    hist = hists[steps % 2]
    torch.cuda.synchronize()
    u_seq = np.stack(us, axis=1)                      # [B][steps][D] stored bf16
    y_seq = torch.stack(ys, dim=1)                    # [B][steps][D]
    streams = [s for s in sample_streams if s < B]
    K = D // H
    for hh in sample_heads:
        sl = slice(hh * K, (hh + 1) * K)
        op = dict(conv_w=synth.widen(params.conv_w)[sl], conv_b=synth.widen(params.conv_b)[sl],
                  W_a=synth.widen(params.W_a)[hh:hh + 1], b_a=synth.widen(params.b_a)[sl],
                  W_x=synth.widen(params.W_x)[hh:hh + 1], b_x=synth.widen(params.b_x)[sl],
                  Lambda=synth.widen(params.Lambda)[sl])
        uo = synth.widen(np.ascontiguousarray(u_seq[streams][:, :, sl]))
        ry, rh, rho = oracle.fwd(uo, **op)
        _cmp(f"y[h={hh}]", from_dev(y_seq[streams][:, :, sl]), ry, TOL["bf16"])
        _cmp(f"h[h={hh}]", from_dev(h[streams][:, sl]), rh, TOL["bf16"])
        got_hist = hist[streams][:, :, sl].cpu().view(torch.int16).numpy().view(np.uint16)
        want = np.ascontiguousarray(u_seq[streams][:, -3:, sl]) if steps >= 3 else None
        if want is not None:
            assert np.array_equal(got_hist, want)
    return u_seq, y_seq, w


def test_decode_short_all_streams():
    _say("decode: B=256 D=2560, 8 steps")
    _decode_run(8)


def test_decode_full_512_steps():
    _say("decode: B=256 D=2560, 512 steps (the decode workload)")
    _decode_run(512)


@pytest.mark.parametrize("B", [45, 130])
def test_decode_ragged_stream_count(B):
    # a partial tile of 64 streams (45), and two full tiles plus a partial one (130)
    _say(f"decode: B={B} (not a multiple of 64), 6 steps")
    _decode_run(6, B=B, sample_streams=(0, 31, 44, 63, 64, 127, 128, 129))


def test_steps_equal_prefill_on_gpu():
    u_seq, y_seq, w = _decode_run(40, B=64, sample_streams=(0,), sample_heads=(3,))
    y, hl, ho = glr.scan_fwd(to_dev(u_seq, DEV), w)
    torch.cuda.synchronize()
    _cmp("steps vs prefill", from_dev(y_seq), from_dev(y), 1e-2)


def test_decode_fp32_tiny_width():
    # fp32 I/O on the tiny workload's parameters (D = 256, one block),
    # 20 streams with a nonzero starting history and state, 10 steps
    cfg = synth.TINY
    B, D, steps = 20, cfg.D, 10
    params = synth.make_params(cfg.idx, D, cfg.H, "f32")
    w = glr.Weights(conv_w=to_dev(params.conv_w, DEV), W_a=to_dev(params.W_a, DEV),
                    W_x=to_dev(params.W_x, DEV), Lambda=to_dev(params.Lambda, DEV),
                    conv_b=to_dev(params.conv_b, DEV), b_a=to_dev(params.b_a, DEV),
                    b_x=to_dev(params.b_x, DEV))
    hist0 = synth.make_activation(cfg.idx, "hist", (B, 3, D), "f32")
    h00 = synth.store(synth.normal(synth.seed_for(cfg.idx, "h0"), 0, B * D), "f32").reshape(B, D)
    u_seq = synth.make_activation(cfg.idx, "u", (B, steps, D), "f32")
    hists = [to_dev(hist0, DEV), torch.empty((B, 3, D), dtype=torch.float32, device=DEV)]
    h = to_dev(h00, DEV)
    _say(f"decode fp32: B={B} D={D}, {steps} steps with history and state")
    ys = []
    for s in range(steps):
        y, _ = glr.step(to_dev(np.ascontiguousarray(u_seq[:, s]), DEV), w, h, hists[s % 2], hists[(s + 1) % 2])
        ys.append(y)
    hist = hists[steps % 2]
    torch.cuda.synchronize()
    op = dict(conv_w=synth.widen(params.conv_w), conv_b=synth.widen(params.conv_b),
              W_a=synth.widen(params.W_a), b_a=synth.widen(params.b_a),
              W_x=synth.widen(params.W_x), b_x=synth.widen(params.b_x),
              Lambda=synth.widen(params.Lambda))
    ry, rh, rho = oracle.fwd(synth.widen(u_seq), **op, h0=h00.astype(np.float64), hist_in=synth.widen(hist0))
    _cmp("y", from_dev(torch.stack(ys, dim=1)), ry, TOL["f32"])
    _cmp("h", from_dev(h), rh, TOL["f32"])
    assert np.array_equal(hist.cpu().numpy(), u_seq[:, -3:, :])


def test_decode_graph_replays_equal_eager():
    # 16 steps captured in a HIP graph: each replay, with eager work and a
    # synchronisation between replays, gives what the eager steps gave
    cfg = synth.DECODE_256
    B, D, H, steps = 64, cfg.D, cfg.H, 16
    params = synth.make_params(cfg.idx, D, H, cfg.io)
    w = glr.Weights(conv_w=to_dev(params.conv_w, DEV), W_a=to_dev(params.W_a, DEV),
                    W_x=to_dev(params.W_x, DEV), Lambda=to_dev(params.Lambda, DEV),
                    conv_b=to_dev(params.conv_b, DEV), b_a=to_dev(params.b_a, DEV),
                    b_x=to_dev(params.b_x, DEV))
    u = to_dev(synth.make_activation(cfg.idx, "u", (steps, B, D), cfg.io), DEV)
    y = torch.empty_like(u)
    h = torch.zeros((B, D), dtype=torch.float32, device=DEV)
    hists = [torch.zeros((B, 3, D), dtype=torch.bfloat16, device=DEV) for _ in range(2)]

    def run():
        for k in range(steps):
            glr.step(u[k], w, h, hists[k % 2], hists[(k + 1) % 2], y[k])

    run()
    torch.cuda.synchronize()
    y_ref, h_ref, hist_ref = y.clone(), h.clone(), hists[steps % 2].clone()
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        with torch.cuda.graph(graph, stream=gs):
            run()
    torch.cuda.current_stream().wait_stream(gs)
    for rep in range(3):
        h.zero_()
        for hb in hists:
            hb.zero_()
        y.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(h, h_ref), f"replay {rep} differs"
        assert torch.equal(hists[steps % 2], hist_ref), f"replay {rep}: history differs"
