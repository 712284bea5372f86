#!/usr/bin/env python
"""Throughput of the RG-LRU hot path on one MI355X.

The headline step is one rglru_scan_fwd call in mode A (causal conv of width 4
+ block-diagonal gates + log-space decay + chunked scan, fused in one kernel)
over one batch of the 2B-width prefill workload: B = 8 streams, T = 2048
tokens, D = 2560 channels (10 blocks of 256), bf16 activations and gate
weights, fp32 state.  Inputs are seeded synthetic data (the generator in
synth/), resident in HBM before timing.  Four input/output buffer sets
(672 MB) rotate so that the 256 MB Infinity Cache cannot serve a step from
the previous one.

The other entry points are timed the same way, each on its own workload, and
reported under "rows": conv1d, gates and the scan stage alone on the 2B-width
prefill, the recurrent block around the path on the same shape (three
projections plus the fused forward with the GeLU merge, d_model = D = 2560),
the residual layer around it (two RMSNorms, the block, a gated GELU-tanh MLP
of width 3 d_model, residual adds),
the fused forward on the 32k-token prefill and on the 9B-width workload
(B = 4, T = 8192, D = 4096), 512 decode steps of 256 streams,
the backward of the 9B-width workload (B = 4, T = 8192, D = 4096), and the
local sliding-window MQA (10 query heads of 256, window 2048) as prefill on
the 2B-width and 32k-token shapes and as a decode step of 256 streams, and
Griffin's attention residual layer around it (projections, rotary embedding,
gated MLP).

Prints ONE JSON line: tokens*channels/s for the whole job, the dominant
kernel's achieved algorithmic HBM bandwidth against the 8 TB/s peak (kernel
durations from HIP events recorded on the launch stream), and the CPU oracle
timed on a bounded sample of the same workload.

`--copy-calibration` instead times a plain 1 GiB device copy; its hardware
counters calibrate FETCH_SIZE / WRITE_SIZE for the traffic figure.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
SETTLE_MS = 100.0   # untimed clock-settle time before the headline's warmup steps
PEAK_BF16_TFLOPS = 2500.0
KERNEL_SOURCES = ("fwd.hip", "common.h", "gatemath.h")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "fwd_fused_2b_prefill_pmc.json")
ALL_ROWS = ("conv1d", "gates", "scan", "block", "layer", "long", "fwd9b", "decode", "bwd", "attn", "attn_long",
            "attn_decode", "attn_layer")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_linear_recurrence_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def fwd_bytes(B, T, D, H, esz):
    """Bytes the fused forward must move: u in, y out, gate weights, per-channel
    parameters (conv taps + bias, b_a, b_x, Lambda), h_last and the conv history."""
    act = 2 * B * T * D * esz
    weights = 2 * H * 256 * 256 * esz
    params = D * (4 + 1 + 1 + 1 + 1) * 4
    return act + weights + params + B * D * 4 + B * 3 * D * esz


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(prob, budget_s: float):
    """Time the oracle (as it stands) on whole (stream, block) slices of the workload."""
    import numpy as np

    import oracle
    import synth
    K = prob["D"] // prob["H"]
    p, u = prob["params"], prob["u"]
    done = 0
    t0 = time.perf_counter()
    slices = [(b, h) for b in range(prob["B"]) for h in range(prob["H"])]
    n = 0
    for b, h in slices:
        sl = slice(h * K, (h + 1) * K)
        op = dict(conv_w=synth.widen(p.conv_w)[sl], conv_b=synth.widen(p.conv_b)[sl],
                  W_a=synth.widen(p.W_a)[h:h + 1], b_a=synth.widen(p.b_a)[sl],
                  W_x=synth.widen(p.W_x)[h:h + 1], b_x=synth.widen(p.b_x)[sl],
                  Lambda=synth.widen(p.Lambda)[sl])
        us = synth.widen(np.ascontiguousarray(u[b:b + 1, :, sl]))
        oracle.fwd(us, **op)
        done += us.size
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    cores = oracle.num_threads()
    # the tiny fp32 configuration (B=1 T=256 D=256) on one thread, for scale
    c0 = synth.TINY
    p0 = synth.make_params(0, c0.D, c0.H, c0.io)
    u0 = synth.widen(synth.make_activation(0, "u", (c0.B, c0.T, c0.D), c0.io))
    op0 = {k: synth.widen(getattr(p0, k)) for k in ("conv_w", "conv_b", "W_a", "b_a", "W_x", "b_x", "Lambda")}
    oracle.set_threads(1)
    try:
        t1 = time.perf_counter()
        reps = 0
        while reps < 3 or time.perf_counter() - t1 < 0.5:
            oracle.fwd(u0, **op0)
            reps += 1
        dt1 = (time.perf_counter() - t1) / reps
    finally:
        oracle.set_threads(cores)
    return dict(value=done / dt, unit="tokens*ch/s", cores=cores, kind="oracle",
                sample=f"{n} of {len(slices)} (stream, 256-channel block) slices of the 2B-width "
                       f"prefill workload ({done} tokens*ch), double precision, {dt:.1f} s",
                single_thread_tiny=dict(value=u0.size / dt1, unit="tokens*ch/s", cores=1,
                                        sample="B=1 T=256 D=256 fp32 configuration, whole, "
                                               f"{dt1 * 1e3:.1f} ms per call"))


class Timer:
    """Per-call durations from HIP events recorded on the launch stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def calls(self, fn, n, warmup):
        torch = self.torch
        for k in range(warmup):
            fn(k)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        t0 = time.perf_counter()
        for k in range(n):
            evs[k][0].record(self.stream)
            fn(k)
            evs[k][1].record(self.stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / n
        return [a.elapsed_time(b) for a, b in evs], wall

    def span(self, fn, n):
        """One event pair around n back-to-back calls; returns ms per call."""
        torch = self.torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for k in range(n):
            fn(k)
        b.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n


def row(workload, kms, tokch, nbytes, flops=None, note=None, bound="hbm"):
    import numpy as np
    ms = float(np.mean(kms)) if isinstance(kms, list) else float(kms)
    r = {"workload": workload, "kernel_ms": ms, "tokens_ch_per_s": tokch / (ms * 1e-3),
         "algorithmic_bytes": nbytes, "achieved_gbs": nbytes / (ms * 1e-3) / 1e9,
         "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bound": bound}
    if isinstance(kms, list):
        r["kernel_ms_min"] = float(np.min(kms))
    if flops is not None:
        r["algorithmic_flops"] = flops
        r["achieved_tflops"] = flops / (ms * 1e-3) / 1e12
        r["mfma_frac_bf16"] = r["achieved_tflops"] / PEAK_BF16_TFLOPS
    if note:
        r["note"] = note
    return r


def copy_calibration(torch, dev, n=10):
    """A plain 1 GiB device copy (torch's copy kernel), timed with HIP events.
    Run under rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE), its per-dispatch
    readings against the known 1 GiB read and written give the scale factors
    that turn the counters of the fused forward into HBM bytes."""
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    tm = Timer(torch, torch.cuda.current_stream(dev))
    kms, _ = tm.calls(lambda k: dst.copy_(src), n, 2)
    import numpy as np
    ms = float(np.mean(kms))
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "calls": n,
                      "kernel_ms": ms, "gbs": 2 * nbytes / (ms * 1e-3) / 1e9}), flush=True)


# kernels that the counter summaries cover: (label, regular expression for the
# kernel name as rocprofv3 reports it, demangled "<__bf16, 0>" or mangled
# "IDF16bLi0E" for the bf16 template arguments)
PROFILED_KERNELS = (
    ("fused forward, mode A (rglru_scan_fwd)", r"(?<![a-z_])fwd_kernel(<__bf16, 0>|IDF16bLi0E)"),
    ("backward pass 1: states, r, i (mode-3 forward)", r"(?<![a-z_])fwd_kernel(<__bf16, 3>|IDF16bLi3E)"),
    ("backward pass 3: reverse aggregates", r"rev_agg_kernel(<__bf16>|IDF16b)"),
    ("backward pass 4: unit kernel", r"bwd_unit_kernel(<__bf16>|IDF16b)"),
    ("backward pass 6: dW", r"dw_kernel_bf16"),
    ("decode step (rglru_step)", r"step_kernel(<__bf16>|IDF16b)"),
)


def summarize(args):
    """Summaries of rocprofv3 output kept in profiles/ (no GPU needed)."""
    from gated_linear_recurrence_02_amd import profiling
    import synth
    if args.summarize_traffic:
        d = args.summarize_traffic
        match = PROFILED_KERNELS[0][1]
        cfg = synth.PREFILL_2B
        t = profiling.traffic(os.path.join(d, "fetch"), os.path.join(d, "write"), os.path.join(d, "copy_fetch"),
                              os.path.join(d, "copy_write"), match, 1 << 30)
        alg = fwd_bytes(cfg.B, cfg.T, cfg.D, cfg.H, 2)
        out = {"kernel": "fwd_kernel<bf16, mode A>",
               "workload": f"2B-width prefill B={cfg.B} T={cfg.T} D={cfg.D} bf16",
               "kernel_source_hash": kernel_hash(),
               "commands": {
                   "fetch": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --kernel-trace "
                            "--output-format csv -d <out>/fetch -- python3 <repo>/bench.py --steps 5 --warmup 1 "
                            "--no-cpu --rows=",
                   "write": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --kernel-trace "
                            "--output-format csv -d <out>/write -- python3 <repo>/bench.py --steps 5 --warmup 1 "
                            "--no-cpu --rows=",
                   "copy_fetch": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --kernel-trace "
                                 "--output-format csv -d <out>/copy_fetch -- python3 <repo>/bench.py "
                                 "--copy-calibration",
                   "copy_write": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --kernel-trace "
                                 "--output-format csv -d <out>/copy_write -- python3 <repo>/bench.py "
                                 "--copy-calibration",
                   "summary": "python3 <repo>/bench.py --summarize-traffic <out>"},
               **t,
               "algorithmic_bytes_per_launch": alg,
               "traffic_over_algorithmic": round(t["hbm_bytes_per_launch"] / alg, 3),
               "note": "FETCH_SIZE/WRITE_SIZE count traffic between L2 and the fabric (Infinity Cache hits "
                       "included); each is scaled by what the same counter reads for torch's copy of 1 GiB. "
                       "kernel_source_hash covers the sources of the kernel; bench.py reports traffic only "
                       "while it matches."}
        print(json.dumps(out, indent=1))
    if args.summarize_counters:
        print(profiling.counter_table(args.summarize_counters, PROFILED_KERNELS))
    if args.summarize_trace:
        print(profiling.trace_table(args.summarize_trace))


def micro(torch, dev):
    """Ceilings on this GPU: vector-ALU rates (FMA and the transcendentals the
    gate math uses), bf16 MFMA rate and plain copy bandwidth, from the kernels
    of librglru_micro.so, each timed with HIP events on the launch stream."""
    import ctypes

    import numpy as np
    path = os.path.join(ROOT, "gated_linear_recurrence_02_amd", "librglru_micro.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built; run gated_linear_recurrence_02_amd/build.py")
    L = ctypes.CDLL(path)
    L.rglru_micro_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.rglru_micro_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.rglru_micro_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                   ctypes.c_void_p]
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    tm = Timer(torch, stream)
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 8 * ncu   # 8 workgroups of 4 waves per CU: 8 waves per SIMD
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    res = {"cus": ncu, "clock_for_cycles_ghz": 2.4}

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"micro kernel launch failed: hip error {rc}")

    iters = 2048
    for kind, name in enumerate(("fma", "exp2", "rcp", "sqrt", "exp2+fma")):
        kms, _ = tm.calls(lambda k: check(L.rglru_micro_valu(kind, blocks, iters, out.data_ptr(), sp)), 5, 2)
        ms = float(np.median(kms))
        wave_instr_per_simd = blocks * 4 * iters * 8 / (ncu * 4)
        ns = ms * 1e6 / wave_instr_per_simd
        res[f"valu_{name}"] = {"lane_ops_per_s": blocks * 256 * iters * 8 / (ms * 1e-3),
                               "ns_per_wave_instr_per_simd": ns, "cycles_at_2p4ghz": ns * 2.4}
    kms, _ = tm.calls(lambda k: check(L.rglru_micro_mfma(blocks, 1024, out.data_ptr(), sp)), 5, 2)
    ms = float(np.median(kms))
    flops = blocks * 4 * 1024 * 4 * 32768
    res["mfma_bf16_32x32x16"] = {"tflops": flops / (ms * 1e-3) / 1e12,
                                 "frac_of_2500": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    # MFMA waves and FMA waves on the same SIMDs: alone and together
    L.rglru_micro_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    mblocks = 2 * ncu
    mout = torch.empty(mblocks * 512, dtype=torch.float32, device=dev)
    mix = {}
    for mode, name in enumerate(("mfma_alone", "fma_alone", "together")):
        kms, _ = tm.calls(lambda k: check(L.rglru_micro_mix(mode, mblocks, 512, 2048, mout.data_ptr(), sp)), 5, 2)
        mix[name + "_ms"] = float(np.median(kms))
    mix["together_over_max"] = mix["together_ms"] / max(mix["mfma_alone_ms"], mix["fma_alone_ms"])
    mix["together_over_sum"] = mix["together_ms"] / (mix["mfma_alone_ms"] + mix["fma_alone_ms"])
    res["mfma_fma_coexecution"] = mix
    # one wave per SIMD issuing its own MFMAs and independent FMAs in one loop
    L.rglru_micro_interleave.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p]
    iblocks = ncu
    iout = torch.empty(iblocks * 256, dtype=torch.float32, device=dev)
    inter = {}
    for fpm in (4, 8, 16):
        r = {}
        for mode, name in enumerate(("mfma_alone", "fma_alone", "together")):
            kms, _ = tm.calls(lambda k: check(L.rglru_micro_interleave(mode, iblocks, 2048, fpm, iout.data_ptr(),
                                                                        sp)), 5, 2)
            r[name + "_ms"] = float(np.median(kms))
        r["together_over_max"] = r["together_ms"] / max(r["mfma_alone_ms"], r["fma_alone_ms"])
        r["together_over_sum"] = r["together_ms"] / (r["mfma_alone_ms"] + r["fma_alone_ms"])
        inter[f"fma_per_4_mfma_{8 * fpm}"] = r
    res["same_wave_interleave_1_wave_per_simd"] = inter
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for cb in (ncu * 4, ncu * 16):
        kms, _ = tm.calls(lambda k: check(L.rglru_micro_copy(src.data_ptr(), dst.data_ptr(), nbytes, cb, sp)),
                          10, 2)
        ms = float(np.median(kms))
        res[f"copy_1gib_{cb}_workgroups"] = {"gbs": 2 * nbytes / (ms * 1e-3) / 1e9,
                                             "frac_of_8000": 2 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    if not torch.equal(src, dst):
        raise RuntimeError("copy microbenchmark: destination differs from source")
    print(json.dumps({"micro": res}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--rows", default=",".join(ALL_ROWS),
                    help="comma-separated extra rows to time (empty for the headline only): "
                         + ",".join(ALL_ROWS))
    ap.add_argument("--micro", action="store_true",
                    help="run the ALU, MFMA and copy microbenchmarks and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 1 GiB device copy and exit")
    ap.add_argument("--summarize-traffic", metavar="DIR",
                    help="print the HBM traffic summary of the headline kernel from rocprofv3 CSV output "
                         "under DIR/fetch, DIR/write (FETCH_SIZE / WRITE_SIZE runs of this script) and "
                         "DIR/copy_fetch, DIR/copy_write (the same runs of --copy-calibration), then exit")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print per-kernel calls and durations from rocprofv3 --kernel-trace --stats CSV "
                         "output under DIR, then exit")
    ap.add_argument("--summarize-counters", metavar="DIR", nargs="+",
                    help="print the per-kernel means of every counter found in rocprofv3 --pmc CSV "
                         "output under the DIRs (one per counter pass), then exit")
    args = ap.parse_args()
    if args.summarize_traffic or args.summarize_counters or args.summarize_trace:
        summarize(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(the library runs on and reports a single MI355X; the sharding plan is "
              f"described but not implemented)", file=sys.stderr)
        sys.exit(2)
    rows = [r for r in args.rows.split(",") if r]
    for r in rows:
        if r not in ALL_ROWS:
            ap.error(f"unknown row {r!r}")

    import numpy as np
    import torch

    import gated_linear_recurrence_02_amd as glr
    import synth

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(torch, dev)
        return
    if args.micro:
        micro(torch, dev)
        return
    glr.lib()
    stream = torch.cuda.current_stream(dev)
    tm = Timer(torch, stream)

    def dev_t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def weights(cfg):
        p = synth.make_params(cfg.idx, cfg.D, cfg.H, cfg.io)
        w = glr.Weights(conv_w=dev_t(p.conv_w), W_a=dev_t(p.W_a), W_x=dev_t(p.W_x),
                        Lambda=dev_t(p.Lambda), conv_b=dev_t(p.conv_b),
                        b_a=dev_t(p.b_a), b_x=dev_t(p.b_x))
        return p, w

    # ------------------------------------------------ headline: fused forward
    cfg = synth.PREFILL_2B
    B, T, D, H = cfg.B, cfg.T, cfg.D, cfg.H
    params, w = weights(cfg)
    u_host = synth.make_u(cfg)
    NSET = 4
    u0 = dev_t(u_host)
    sets = []
    for _ in range(NSET):
        sets.append(dict(u=u0.clone(), y=torch.empty_like(u0),
                         h=torch.empty((B, D), dtype=torch.float32, device=dev),
                         hist=torch.empty((B, 3, D), dtype=torch.bfloat16, device=dev)))
    del u0
    # workspace allocated once, before timing
    glr.workspace(glr.workspace_size(B, T, D, H, glr.BF16, glr.OP_SCAN_FWD), dev)

    def step(k):
        s = sets[k % NSET]
        glr.scan_fwd(s["u"], w, out=s["y"], h_last_out=s["h"], hist_out_buf=s["hist"])

    _say(f"fused forward, 2B-width prefill B={B} T={T} D={D}: {args.warmup} warmup + {args.steps} timed")
    # clock settle: after the host-side set-up the GPU has been idle and runs
    # at a low clock for the first milliseconds of load (5 back-to-back steps
    # measured 138 us per step, the same steps after 200 others 123 us), so
    # the same step is launched, untimed, for SETTLE_MS of wall time before
    # the warmup steps; the JSON line reports it under "settle"
    t_set = time.perf_counter()
    n_settle = 0
    while (time.perf_counter() - t_set) * 1e3 < SETTLE_MS:
        step(n_settle)
        n_settle += 1
        if n_settle % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    settle = {"ms": round((time.perf_counter() - t_set) * 1e3, 1), "launches": n_settle,
              "note": "untimed launches of the headline step before the warmup steps, to bring the GPU "
                      "clocks to their loaded state"}
    # the step rate: K steps back to back, synchronised on both sides
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # the kernel's own duration: the same steps again, each between two events
    kms, _ = tm.calls(step, args.steps, 0)
    kernel_ms = float(np.mean(kms))
    tokch = B * T * D
    alg = fwd_bytes(B, T, D, H, 2)
    achieved = alg / (kernel_ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(PMC_SUMMARY):
        pmc = json.load(open(PMC_SUMMARY))
        if pmc.get("kernel_source_hash") == kernel_hash():
            traffic = pmc.get("hbm_bytes_per_launch")

    out = {
        "metric": "RG-LRU fwd scan tokens·ch/s + achieved HBM GB/s (% of peak), 2B width",
        "value": tokch / (ms_per_step * 1e-3),
        "unit": "tokens·ch/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settle,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller; u ~ N(0,1), conv taps N(0,1/4), "
                "gate weights N(0,1/256), a^8 ~ U[0.9,0.999])",
        "config": {"workload": "2B-width prefill: fused conv(k=4) + RG-LRU forward scan (mode A)",
                   "B": B, "T": T, "D": D, "H": H, "K": 256, "io": "bf16", "state": "fp32",
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "kernel_ms": kernel_ms,
        "kernel_ms_min": float(np.min(kms)),
        "kernel_tokens_ch_per_s": tokch / (kernel_ms * 1e-3),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "fwd_kernel<bf16, mode A>",
                     "algorithmic_bytes_per_launch": alg},
        "rows": {},
    }

    # ------------------------------------------------ other rows
    if "conv1d" in rows or "gates" in rows or "scan" in rows:
        for s in sets:
            s["x"] = torch.empty_like(s["u"])
            glr.conv1d(s["u"], w.conv_w, w.conv_b, H=H, out=s["x"], hist_out_buf=s["hist"])
        if "conv1d" in rows:
            _say("conv1d alone, 2B-width prefill")
            kk, _ = tm.calls(lambda k: glr.conv1d(sets[k % NSET]["u"], w.conv_w, w.conv_b, H=H,
                                                  out=sets[k % NSET]["x"],
                                                  hist_out_buf=sets[k % NSET]["hist"]), 20, 3)
            nb = 2 * tokch * 2 + B * 3 * D * 2 + D * 5 * 4
            out["rows"]["conv1d"] = row("rglru_conv1d, 2B-width prefill (B=8 T=2048 D=2560 bf16)",
                                        kk, tokch, nb)
        if "gates" in rows or "scan" in rows:
            for s in sets[:2]:
                s["r"], s["i"] = torch.empty_like(s["u"]), torch.empty_like(s["u"])
        if "gates" in rows:
            _say("gates alone, 2B-width prefill")
            kk, _ = tm.calls(lambda k: glr.gates(sets[k % 2]["x"], w, sets[k % 2]["r"],
                                                 sets[k % 2]["i"]), 20, 3)
            nb = 3 * tokch * 2 + 2 * H * 65536 * 2 + 2 * D * 4
            out["rows"]["gates"] = row("rglru_gates, 2B-width prefill (B=8 T=2048 D=2560 bf16)",
                                       kk, tokch, nb, flops=2 * 2 * 256 * tokch, bound="hbm+mfma")
        if "scan" in rows:
            for s in sets[:2]:
                glr.gates(s["x"], w, s["r"], s["i"])
            wc = glr.Weights(conv_w=None, W_a=None, W_x=None, Lambda=w.Lambda)
            _say("scan stage alone (mode C), 2B-width prefill")
            kk, _ = tm.calls(lambda k: glr.scan_fwd(sets[k % 2]["x"], wc, r=sets[k % 2]["r"],
                                                    i=sets[k % 2]["i"], out=sets[k % 2]["y"],
                                                    h_last_out=sets[k % 2]["h"]), 20, 3)
            nb = 4 * tokch * 2 + D * 4 + B * D * 4
            out["rows"]["scan"] = row("rglru_scan_fwd mode C (x, r, i given), 2B-width prefill",
                                      kk, tokch, nb)
        for s in sets:
            for key in ("x", "r", "i"):
                s.pop(key, None)
    del sets
    torch.cuda.empty_cache()

    if "block" in rows:
        # the recurrent block around the path: two input projections, the fused
        # forward with the GeLU merge (mode 4), the output projection
        dm = D
        bp = synth.make_block_params(cfg.idx, dm, D, cfg.io)
        bw = glr.BlockWeights(dev_t(bp.proj_in_1), dev_t(bp.proj_in_2), dev_t(bp.proj_out))
        x0 = dev_t(synth.make_activation(cfg.idx, "block_x", (B, T, dm), cfg.io))
        b_sets = [dict(x=x0 if k == 0 else x0.clone(), o=torch.empty_like(x0)) for k in range(2)]
        hb = torch.empty((B, D), dtype=torch.float32, device=dev)
        sb = torch.empty((B, 3, D), dtype=torch.bfloat16, device=dev)
        glr.workspace(glr.block_workspace_size(B, T, D, H, dm, glr.BF16), dev, "block",
                      (B, T, D, H, dm, glr.BF16))
        _say(f"recurrent block, 2B width B={B} T={T} D=d_model={D}")

        def bstep(k):
            s = b_sets[k % 2]
            glr.block_fwd(s["x"], w, bw, out=s["o"], h_last_out=hb, hist_out_buf=sb)
        kk, _ = tm.calls(bstep, 20, 3)
        M = B * T
        gemm_flops = 3 * 2 * M * dm * D
        # algorithmic bytes: x in, out, the three projections, the RG-LRU's own
        # parameters, state and history (b1, b2 and the merged product are the
        # block's intermediates)
        nb = 2 * M * dm * 2 + 3 * D * dm * 2 + 2 * H * 65536 * 2 + D * 8 * 4 + B * D * 4 + B * 3 * D * 2
        r = row(f"rglru_block_fwd, 2B width (B={B} T={T} D=d_model={D} bf16): 3 projections "
                "(hand-written MFMA GEMM) + fused forward with the GeLU merge", kk, tokch, nb,
                flops=gemm_flops + 2 * 2 * 256 * tokch, bound="mfma",
                note="algorithmic flops: the three projections (3 x 2 M d_model D) and the gate "
                     "products; tokens_ch counts B*T*D")
        # the same three products through torch (hipBLASLt/rocBLAS as torch picks), for context
        import torch.nn.functional as F
        zt = torch.empty((B, T, D), dtype=torch.bfloat16, device=dev)

        def tstep(k):
            s = b_sets[k % 2]
            F.linear(s["x"], bw.proj_in_1)
            F.linear(s["x"], bw.proj_in_2)
            F.linear(zt, bw.proj_out)
        tk, _ = tm.calls(tstep, 10, 2)
        r["torch_linear_x3_ms"] = float(np.mean(tk))
        out["rows"]["block"] = r
        del b_sets, x0, zt, bw
        torch.cuda.empty_cache()

    if "layer" in rows:
        # the residual layer around the block: pre-norms, the block with its
        # residual add, the gated MLP (d_ff = 3 d_model) with its residual add
        dm, F = D, 3 * D
        bp = synth.make_block_params(cfg.idx, dm, D, cfg.io)
        lp = synth.make_layer_params(cfg.idx, dm, F, cfg.io)
        bw = glr.BlockWeights(dev_t(bp.proj_in_1), dev_t(bp.proj_in_2), dev_t(bp.proj_out))
        lw = glr.LayerWeights(dev_t(lp.tnorm_w), dev_t(lp.cnorm_w), dev_t(lp.gate_w), dev_t(lp.up_w),
                              dev_t(lp.down_w))
        x0 = dev_t(synth.make_activation(cfg.idx, "block_x", (B, T, dm), cfg.io))
        l_sets = [dict(x=x0 if k == 0 else x0.clone(), o=torch.empty_like(x0)) for k in range(2)]
        hb = torch.empty((B, D), dtype=torch.float32, device=dev)
        sb = torch.empty((B, 3, D), dtype=torch.bfloat16, device=dev)
        glr.workspace(glr.layer_workspace_size(B, T, D, H, dm, lw, glr.BF16), dev, "layer",
                      (B, T, D, H, dm, F, glr.BF16))
        _say(f"residual layer, 2B width B={B} T={T} d_model={dm} d_ff={F}")

        def lystep(k):
            s_ = l_sets[k % 2]
            glr.layer_fwd(s_["x"], w, bw, lw, out=s_["o"], h_last_out=hb, hist_out_buf=sb)
        kk, _ = tm.calls(lystep, 10, 2)
        M = B * T
        fl = 3 * 2 * M * dm * D + 2 * 2 * 256 * tokch + 3 * 2 * M * dm * F
        nb = 2 * M * dm * 2 + (3 * D * dm + 3 * F * dm) * 2 + 2 * H * 65536 * 2 + D * 8 * 4 + 2 * dm * 4
        out["rows"]["layer"] = row(f"rglru_layer_fwd, residual layer at 2B width (B={B} T={T} d_model={dm} "
                                   f"d_ff={F} bf16): 2 RMSNorms, block, gated MLP, residual adds", kk, tokch,
                                   nb, flops=fl, bound="mfma",
                                   note="algorithmic flops: 6 projections (block 3, MLP 3) and the gate "
                                        "products; tokens_ch counts B*T*D")
        del l_sets, x0, bw, lw
        torch.cuda.empty_cache()

    if "long" in rows:
        c2 = synth.PREFILL_32K
        _, w2 = weights(c2)
        u2 = dev_t(synth.make_u(c2))
        l_sets = [dict(u=u2 if k == 0 else u2.clone(), y=torch.empty_like(u2),
                       h=torch.empty((c2.B, c2.D), dtype=torch.float32, device=dev),
                       hist=torch.empty((c2.B, 3, c2.D), dtype=torch.bfloat16, device=dev))
                  for k in range(2)]
        glr.workspace(glr.workspace_size(c2.B, c2.T, c2.D, c2.H, glr.BF16, glr.OP_SCAN_FWD), dev)
        _say(f"fused forward, long prefill T={c2.T}")

        def lstep(k):
            s = l_sets[k % 2]
            glr.scan_fwd(s["u"], w2, out=s["y"], h_last_out=s["h"], hist_out_buf=s["hist"])
        kk, _ = tm.calls(lstep, 20, 3)
        t2 = c2.B * c2.T * c2.D
        out["rows"]["long"] = row(f"rglru_scan_fwd mode A, long prefill (B=1 T={c2.T} D={c2.D} bf16)",
                                  kk, t2, fwd_bytes(c2.B, c2.T, c2.D, c2.H, 2))
        del l_sets, u2
        torch.cuda.empty_cache()

    if "fwd9b" in rows:
        c4 = synth.FWD_BWD_9B
        _, w4 = weights(c4)
        u4 = dev_t(synth.make_u(c4))
        f_sets = [dict(u=u4 if k == 0 else u4.clone(), y=torch.empty_like(u4),
                       h=torch.empty((c4.B, c4.D), dtype=torch.float32, device=dev),
                       hist=torch.empty((c4.B, 3, c4.D), dtype=torch.bfloat16, device=dev))
                  for k in range(2)]
        glr.workspace(glr.workspace_size(c4.B, c4.T, c4.D, c4.H, glr.BF16, glr.OP_SCAN_FWD), dev)
        _say(f"fused forward, 9B width B={c4.B} T={c4.T} D={c4.D}")

        def f4step(k):
            s = f_sets[k % 2]
            glr.scan_fwd(s["u"], w4, out=s["y"], h_last_out=s["h"], hist_out_buf=s["hist"])
        kk, _ = tm.calls(f4step, 20, 3)
        t4 = c4.B * c4.T * c4.D
        out["rows"]["fwd9b"] = row(f"rglru_scan_fwd mode A, 9B width (B={c4.B} T={c4.T} D={c4.D} bf16)",
                                   kk, t4, fwd_bytes(c4.B, c4.T, c4.D, c4.H, 2),
                                   flops=2 * 2 * 256 * t4)
        del f_sets, u4
        torch.cuda.empty_cache()

    if "decode" in rows:
        c3 = synth.DECODE_256
        _, w3 = weights(c3)
        n3 = c3.B * c3.D
        # the decode stream [steps][B][D]; call k reads the slice synth.make_decode_u(c3, k)
        u_all = dev_t(synth.make_activation(c3.idx, "u", (c3.steps, c3.B, c3.D), c3.io))
        y_all = torch.empty_like(u_all)
        h = torch.zeros((c3.B, c3.D), dtype=torch.float32, device=dev)
        hists = [torch.zeros((c3.B, 3, c3.D), dtype=torch.bfloat16, device=dev) for _ in range(2)]

        def dstep(k):   # the history alternates between two buffers
            glr.step(u_all[k], w3, h, hists[k % 2], hists[(k + 1) % 2], y_all[k])

        _say(f"decode: {c3.steps} steps of B={c3.B} D={c3.D}")
        for k in range(8):
            dstep(k)
        h.zero_()
        for hb in hists:
            hb.zero_()
        torch.cuda.synchronize()
        ms_eager = tm.span(dstep, c3.steps)
        # the same 512 steps captured once in a HIP graph and replayed: the
        # GPU's own time per step, without the host's per-call cost
        h.zero_()
        for hb in hists:
            hb.zero_()
        torch.cuda.synchronize()
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            with torch.cuda.graph(graph, stream=gs):
                for k in range(c3.steps):
                    dstep(k)
        torch.cuda.current_stream().wait_stream(gs)
        graph.replay()
        torch.cuda.synchronize()
        ms = tm.span(lambda k: graph.replay(), 5) / c3.steps
        nb = n3 * (2 + 2 + 4 * 2 + 3 * 2 * 2) + 2 * c3.H * 65536 * 2 + c3.D * 8 * 4
        out["rows"]["decode"] = row(f"rglru_step, {c3.steps} consecutive calls of B={c3.B} D={c3.D} bf16 "
                                    f"(time per call, the 512 calls replayed as one HIP graph)", ms, n3, nb,
                                    note="state, history and weights (15.7 MB) stay resident in "
                                         "L2/Infinity Cache between calls; eager back-to-back calls from "
                                         "Python, bound by the host: %.1f us per call" % (ms_eager * 1e3))
        out["rows"]["decode"]["eager_ms_per_call"] = ms_eager
        del graph
        del u_all, y_all, h, hists
        torch.cuda.empty_cache()

    if "bwd" in rows:
        c4 = synth.FWD_BWD_9B
        _, w4 = weights(c4)
        u4 = dev_t(synth.make_u(c4))
        dy4 = dev_t(synth.make_dy(c4))
        glr.workspace(glr.workspace_size(c4.B, c4.T, c4.D, c4.H, glr.BF16, glr.OP_SCAN_BWD), dev, "bwd",
                      (c4.B, c4.T, c4.D, c4.H, glr.BF16))
        _say(f"backward, 9B width B={c4.B} T={c4.T} D={c4.D}")
        kk, _ = tm.calls(lambda k: glr.scan_bwd(u4, w4, dy4), 5, 2)
        t4 = c4.B * c4.T * c4.D
        nb = 3 * t4 * 2 + 2 * c4.H * 65536 * (2 + 4) + c4.D * (4 + 1 + 1 + 1 + 1) * 4 * 2
        out["rows"]["bwd"] = row(f"rglru_scan_bwd, 9B width (B={c4.B} T={c4.T} D={c4.D} bf16), "
                                 "all passes", kk, t4, nb, flops=3 * 2 * 2 * 256 * t4,
                                 bound="mfma",
                                 note="algorithmic flops: the gate products of the state pass, "
                                      "dX and dW (3 x 1024 per token*ch); executed MFMA work is "
                                      "larger (split-bf16 operands)")
        del u4, dy4
        torch.cuda.empty_cache()

    # ------------------------------------------------ local sliding-window MQA
    # 10 query heads of 256 (Hq * dh = D = 2560), one key/value head, window 2048
    AH, ADH, AW = 10, 256, 2048

    def attn_flops(Bq, Tq):
        # 4 dh flops per (query row, key in its window): q.k and p v
        keys = sum(min(t + 1, AW) for t in range(Tq))
        return 4 * ADH * AH * Bq * keys

    for name, (Bq, Tq) in (("attn", (B, T)), ("attn_long", (1, 32768))):
        if name not in rows:
            continue
        qa = dev_t(synth.make_activation(30, "attn_q", (Bq, Tq, AH, ADH), "bf16"))
        ka = dev_t(synth.make_activation(30, "attn_k", (Bq, Tq, ADH), "bf16"))
        va = dev_t(synth.make_activation(30, "attn_v", (Bq, Tq, ADH), "bf16"))
        oa = torch.empty_like(qa)
        _say(f"local attention prefill B={Bq} T={Tq} Hq={AH} dh={ADH} W={AW}")
        kk, _ = tm.calls(lambda k: glr.attn_fwd(qa, ka, va, AW, 1.0 / 16, out=oa), 10, 2)
        fl = attn_flops(Bq, Tq)
        nb = 2 * qa.numel() * 2 + 2 * ka.numel() * 2
        out["rows"][name] = row(f"rglru_attn_fwd, sliding-window MQA prefill (B={Bq} T={Tq} Hq={AH} dh={ADH} "
                                f"W={AW} bf16)", kk, Bq * Tq * AH * ADH, nb, flops=fl, bound="mfma",
                                note="algorithmic flops 4*dh per (query row, key in window); tokens_ch "
                                     "counts B*T*Hq*dh outputs")
        del qa, ka, va, oa
        torch.cuda.empty_cache()

    if "attn_decode" in rows:
        Bd = 256
        kc = dev_t(synth.make_activation(31, "attn_hk", (Bd, AW, ADH), "bf16"))
        vc = dev_t(synth.make_activation(31, "attn_hv", (Bd, AW, ADH), "bf16"))
        qd = dev_t(synth.make_activation(31, "attn_q", (64, Bd, AH, ADH), "bf16"))
        kd = dev_t(synth.make_activation(31, "attn_k", (64, Bd, ADH), "bf16"))
        vd = dev_t(synth.make_activation(31, "attn_v", (64, Bd, ADH), "bf16"))
        od = torch.empty((Bd, AH, ADH), dtype=torch.bfloat16, device=dev)
        pos = torch.full((Bd,), 4096, dtype=torch.int32, device=dev)   # every window full
        glr.workspace(glr.attn_workspace_size(Bd, AH, ADH, AW), dev, "attn")
        _say(f"local attention decode B={Bd} W={AW} Hq={AH} dh={ADH}")
        kk, _ = tm.calls(lambda k: glr.attn_step(qd[k % 64], kd[k % 64], vd[k % 64], kc, vc, pos, 1.0 / 16,
                                                 out=od), 30, 3)
        nb = Bd * AW * ADH * 2 * 2 + 2 * Bd * AH * ADH * 2 + 4 * Bd * ADH * 2
        out["rows"]["attn_decode"] = row(f"rglru_attn_step, sliding-window MQA decode (B={Bd}, ring of {AW}, "
                                         f"Hq={AH} dh={ADH} bf16, full windows), per call", kk, Bd * AH * ADH,
                                         nb, note="bytes: the whole ring of keys and values read once, q_t, "
                                                  "o_t, the new key/value written; two launches (splits, "
                                                  "combine)")
        del kc, vc, qd, kd, vd, od
        torch.cuda.empty_cache()

    if "attn_layer" in rows:
        # Griffin's attention residual layer at the 2B width: q/k/v projections,
        # rotary embedding on half of each head (partial rotary), the local
        # MQA, output projection with the residual, gated MLP (d_ff = 3 d_model)
        dm, F = D, 3 * D
        ap = synth.make_attn_proj(cfg.idx, dm, AH, ADH, cfg.io)
        lp = synth.make_layer_params(cfg.idx, dm, F, cfg.io)
        apd = glr.AttnProjWeights(dev_t(ap.wq), dev_t(ap.wk), dev_t(ap.wv), dev_t(ap.wo))
        lw = glr.LayerWeights(dev_t(lp.tnorm_w), dev_t(lp.cnorm_w), dev_t(lp.gate_w), dev_t(lp.up_w),
                              dev_t(lp.down_w))
        x0 = dev_t(synth.make_activation(cfg.idx, "block_x", (B, T, dm), cfg.io))
        a_sets = [dict(x=x0 if k == 0 else x0.clone(), o=torch.empty_like(x0)) for k in range(2)]
        _say(f"attention residual layer, 2B width B={B} T={T} Hq={AH} dh={ADH} W={AW} d_ff={F}")
        kk, _ = tm.calls(lambda k: glr.attn_layer_fwd(a_sets[k % 2]["x"], apd, lw, AH, AW, scale=1.0 / 16,
                                                      rot=ADH // 2, out=a_sets[k % 2]["o"]), 10, 2)
        M = B * T
        fl = 2 * M * dm * (AH * ADH + 2 * ADH) + 2 * M * AH * ADH * dm + attn_flops(B, T) + 3 * 2 * M * dm * F
        nb = 2 * M * dm * 2 + (AH * ADH * dm * 2 + 2 * ADH * dm + 3 * F * dm) * 2 + 2 * dm * 4
        out["rows"]["attn_layer"] = row(f"rglru_attn_layer_fwd, attention residual layer at 2B width (B={B} "
                                        f"T={T} Hq={AH} dh={ADH} W={AW} d_ff={F} bf16)", kk, M * dm, nb,
                                        flops=fl, bound="mfma",
                                        note="algorithmic flops: q/k/v/o and MLP projections and the "
                                             "windowed attention; tokens_ch counts B*T*d_model")
        del a_sets, x0, apd, lw
        torch.cuda.empty_cache()

    if not args.no_cpu:
        _say(f"CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(dict(B=B, T=T, D=D, H=H, params=params, u=u_host),
                                           args.cpu_seconds)
        # the whole-job rate over the oracle's, both on the headline workload
        out["cpu_baseline"]["gpu_over_oracle"] = out["value"] / out["cpu_baseline"]["value"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
