#!/usr/bin/env python3
"""Throughput of the W8A8 INT8 linear layer on one MI355X.

Headline (the JSON `value`): the prefill linear of a 7B-like MLP up-projection,
4096 tokens x (4096 -> 11008), bf16 activations quantized per token on the
fly, INT8 MFMA GEMM, fused dequant epilogue to bf16 -- one step is one whole
prefill linear (quantize + GEMM + epilogue) and `value` is 2*M*N*K / step
time in TOPS.  `roofline` is the INT8 GEMM kernel alone, timed with HIP
events on the stream it is launched on, against the chip's dense INT8 peak.

Also measured in the same run and reported under "prefill_asym", "decode" and
"llm_int8": the same prefill linear with per-token asymmetric activations
(the prefill formula with its per-token zero point), the static per-tensor
decode linear 4096 -> 4096 at M in {1, 8, 32, 64}
(HBM GB/s of the skinny GEMM against 8 TB/s, weights rotated over >= 1 GiB of
copies so that no cache serves them), and the LLM.int8() decomposition
2048 x (8192 -> 28672) in fp16 with threshold 6.0; and under "decoder_block"
the block's four linears (QKV, O, gate+up, down at hidden 4096) on one shared
INT8 weight copy each: a prefill pass over 8192 tokens and 256 decode steps
at batch 32; under "silu_mul_quant" the down projection's input SiLU(gate) * up
(8192 x 14336) quantized by the fused kernel, against the unfused pair, and the
whole down projection; under "cs_cg" the quantizer and GEMM costs (C_s, C_g)
of per-token dynamic against per-tensor static activations at M = 1, 64,
512, 4096 on the decode linear.

Every timed region that follows host-side setup is preceded by 200 ms of
untimed work of its own kind (the clock ramps up over the first ~35 ms after
the GPU idles); "cold_start" reports the headline step timed without it.

cpu_baseline: the CPU oracle timed on the host: whole prefill linears (its
`value`), the linear stage by stage, the decode linear at M = 1 .. 64, the
LLM.int8() layer, and one-thread times of the tiny and M = 1 workloads.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill W8A8 GEMM TOPS + decode GB/s, as % of MI355X INT8/HBM roofline"
PEAK_INT8_TOPS = 5000.0   # MI355X dense INT8 MFMA, published (5.0 POP/s)
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, published (8 TB/s)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_i8_prefill_4096x4096x11008_traffic.json")
GEMM_SRC = os.path.join(ROOT, "w8a8_int8_quantized_absmax_amd", "csrc", "gemm_i8.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed(fn, iters: int, warmup: int, stream) -> float:
    """Average milliseconds per call of fn(i) over `iters` calls, HIP events on `stream`."""
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(iters):
        fn(i)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / iters


def graph_timed(fn, calls: int, replays: int, stream) -> float:
    """Average milliseconds per call of fn(i), i < calls, captured into one HIP
    graph and replayed `replays` times: the launches then go back to back
    without the host's per-call overhead (a few microseconds of Python and
    ctypes that would otherwise starve the GPU between ~5 us kernels)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(replays):
        g.replay()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / (replays * calls)
    del g
    return ms


SETTLE_MS = 200.0  # untimed work before a timed region that follows host-side setup


def settle(fn, stream, ms: float = SETTLE_MS) -> int:
    """Run fn(i) untimed for about `ms` milliseconds of GPU time.

    After the GPU has been idle (here: while the host generates the next
    workload's inputs), the first ~35 ms of back-to-back launches run up to
    30% slower while the power management raises the clock (measured: the
    prefill GEMM 190-250 us over its first ~200 launches after a pause of 1-3
    s, 160-163 us after; the same on the same buffers, so no first-touch
    effect).  Every timed region that follows host-side work is preceded by
    this, so that it measures the steady state; the cold-start figure is
    reported separately."""
    import torch

    t0, n = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


def sample_sclk(fn, ms: float = 600.0):
    """Shader clock (MHz) that rocm-smi reports while fn(i) runs back to back
    for about `ms` milliseconds (untimed; None where rocm-smi is unavailable)."""
    import re
    import subprocess
    import threading

    import torch

    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                                     timeout=5).stdout
                m = re.search(r"sclk clock level:\s*\d+:\s*\((\d+)\s*Mhz\)", out)
                if m:
                    samples.append(int(m.group(1)))
            except Exception:
                return

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0, n = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=6)
    if not samples:
        return None
    samples.sort()
    return {"median_MHz": samples[len(samples) // 2], "min_MHz": samples[0], "max_MHz": samples[-1],
            "samples": len(samples)}


def kernel_hash() -> str:
    """Hash of the GEMM source with its // comments and blank lines removed, so
    that a change of comments alone does not invalidate the counter summary."""
    import re

    with open(GEMM_SRC, encoding="utf-8") as f:
        lines = [re.sub(r"\s*//.*$", "", ln).rstrip() for ln in f]
    code = "\n".join(ln for ln in lines if ln)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_for(per_launch_bytes_expected: float):
    """HBM bytes per GEMM launch from the committed PMC summary, if it is for this kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_hash():
        return None
    return t.get("bytes_per_launch")


def bench_prefill(args, torch, pdq, synth):
    c = synth.Prefill7B()
    M, K, N = c.M, c.K, c.N
    log(f"[prefill] generating X[{M},{K}] and W[{N},{K}] ({c.dtype})")
    x_host, w_host = c.x(), c.w()
    x = torch.from_numpy(x_host).to(torch.bfloat16).cuda()
    wq0, ws, cs = pdq.quantize_weight(torch.from_numpy(w_host).to(torch.bfloat16).cuda())
    nrot = 8  # 8 x 45 MB of INT8 weights + 8 x 34 MB of activations: more than the 256 MB MALL
    wqs = [wq0] + [wq0.clone() for _ in range(nrot - 1)]
    xs = [x] + [x.clone() for _ in range(nrot - 1)]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    xq = torch.empty(pdq.act_bytes(M, K), dtype=torch.int8, device="cuda")  # packed codes
    xsc = torch.empty(M, dtype=torch.float32, device="cuda")
    xqs = [xq] + [xq.clone() for _ in range(nrot - 1)]
    stream = torch.cuda.current_stream()

    def step(i):
        r = i % nrot
        pdq._call("pdq_linear_prefill", pdq._p(xs[r]), pdq.BF16, M, K, K, pdq._p(wqs[r]), pdq._p(ws),
                  None, N, pdq._p(xqs[r]), pdq._p(xsc), pdq._p(y), N, None, pdq._stream(x.device))

    settle(step, stream)
    ms_step = timed(step, args.steps, args.warmup, stream)

    # the INT8 GEMM kernel alone (same launch configuration as inside the step)
    for r in range(nrot):
        pdq.quantize_per_token(xs[r], xq=xqs[r], x_scale=xsc)

    def gemm(i):
        r = i % nrot
        pdq._call("pdq_gemm_per_token", pdq._p(xqs[r]), pdq._p(xsc), M, K, pdq._p(wqs[r]), pdq._p(ws),
                  None, N, pdq._p(y), N, None, pdq._stream(x.device))

    ms_gemm = timed(gemm, args.steps, args.warmup, stream)

    def quant(i):
        r = i % nrot
        pdq._call("pdq_quantize_per_token", pdq._p(xs[r]), pdq.BF16, M, K, K, pdq._p(xqs[r]),
                  pdq._p(xsc), pdq._stream(x.device))

    ms_quant = timed(quant, args.steps, args.warmup, stream)

    # the per-token asymmetric variant (prefill formula with Z_token): the
    # composite call, its quantizer and its GEMM, on the same operands
    xz = torch.empty(M, dtype=torch.int32, device="cuda")

    def step_asym(i):
        r = i % nrot
        pdq._call("pdq_linear_prefill_asym", pdq._p(xs[r]), pdq.BF16, M, K, K, pdq._p(wqs[r]), pdq._p(ws),
                  pdq._p(cs), None, N, pdq._p(xqs[r]), pdq._p(xsc), pdq._p(xz), pdq._p(y), N, None,
                  pdq._stream(x.device))

    def quant_asym(i):
        r = i % nrot
        pdq._call("pdq_quantize_per_token_asym", pdq._p(xs[r]), pdq.BF16, M, K, K, pdq._p(xqs[r]),
                  pdq._p(xsc), pdq._p(xz), pdq._stream(x.device))

    def gemm_asym(i):
        r = i % nrot
        pdq._call("pdq_gemm_per_token_asym", pdq._p(xqs[r]), pdq._p(xsc), pdq._p(xz), M, K, pdq._p(wqs[r]),
                  pdq._p(ws), pdq._p(cs), None, N, pdq._p(y), N, None, pdq._stream(x.device))

    # Context, not part of the step: the vendor library's INT8 GEMM (hipBLASLt
    # through torch._int_mm, INT32 output, no quantization or epilogue) on the
    # same codes in row-major form, rotated over the same number of copies.
    ms_lib = None
    try:
        a_rm = torch.from_numpy(pdq.Codes(xqs[0], M, K).unpack()).cuda()
        b_rm = torch.from_numpy(pdq.unpack(wq0, N, K)).cuda()
        bs = [b_rm] + [b_rm.clone() for _ in range(nrot - 1)]

        def lib_gemm(i):
            torch._int_mm(a_rm, bs[i % nrot].t())

        settle(lib_gemm, stream)  # after the host-side unpacking above
        ms_lib = timed(lib_gemm, max(args.steps // 2, 10), args.warmup // 2, stream)
        del bs, a_rm, b_rm
    except (RuntimeError, TypeError) as e:  # no hipBLASLt INT8 path for this shape or build
        log(f"[prefill] torch._int_mm reference unavailable: {e}")

    asym_steps = max(args.steps // 2, 10)
    settle(step_asym, stream)
    ms_step_asym = timed(step_asym, asym_steps, args.warmup // 2, stream)
    ms_quant_asym = timed(quant_asym, asym_steps, args.warmup // 2, stream)
    for r in range(nrot):  # codes, scales and zero points of every activation copy
        quant_asym(r)
    ms_gemm_asym = timed(gemm_asym, asym_steps, args.warmup // 2, stream)
    for r in range(nrot):  # symmetric codes again for the GEMM-only figures below
        pdq.quantize_per_token(xs[r], xq=xqs[r], x_scale=xsc)
    # the shader clock while the GEMM runs back to back (untimed)
    sclk = sample_sclk(gemm)
    # cold start: the same step timed as above but right after the GPU has
    # been idle for 1.5 s, without the settling phase
    torch.cuda.synchronize()
    time.sleep(1.5)
    ms_step_cold = timed(step, args.steps, args.warmup, stream)
    # one untimed call with the INT32 accumulators: its outputs, on the host,
    # for the CPU-baseline leg to compare with the oracle's same linear
    chk = pdq.linear_prefill(x, wq0, ws, want_acc=True)
    torch.cuda.synchronize()
    gpu_out = dict(xq=chk["xq"].unpack(), x_scale=chk["x_scale"].cpu().numpy(), acc=chk["acc"].cpu().numpy(),
                   y=chk["y"].cpu().view(torch.int16).numpy().view(np.uint16))
    del chk
    ops = 2.0 * M * N * K
    gemm_tops = ops / (ms_gemm * 1e-3) / 1e12
    gemm_bytes = M * K + N * K + 4 * (M + N) + 2 * M * N  # xq, wq, scales, bf16 y
    quant_bytes = 2 * M * K + M * K + 4 * M
    del wqs, xs, xqs
    return dict(M=M, K=K, N=N, ms_step=ms_step, ms_gemm=ms_gemm, ms_quant=ms_quant, ops=ops,
                ms_step_cold=ms_step_cold, sclk=sclk,
                ms_step_asym=ms_step_asym, ms_quant_asym=ms_quant_asym, ms_gemm_asym=ms_gemm_asym,
                ms_lib=ms_lib,
                gemm_tops=gemm_tops, gemm_bytes=gemm_bytes, quant_bytes=quant_bytes,
                x_host=x_host, w_host=w_host, gpu_out=gpu_out)


def bench_decode(args, torch, pdq, synth):
    c = synth.Decode()
    K, N = c.K, c.N
    log(f"[decode] calibrating on {c.n_calib} batches of [{c.calib_tokens},{K}]")
    mm = pdq.minmax_state("cuda")
    for b in range(c.n_calib):
        out = pdq.calibrate_static(torch.from_numpy(c.calib(b)).to(torch.bfloat16).cuda(), mm,
                                   finalize=b == c.n_calib - 1)
    s_t, z_t = out
    s, z = float(s_t.item()), int(z_t.item())
    # the static tensor-wise symmetric variant's scale from the same batches
    mm_sym = pdq.minmax_state("cuda")
    for b in range(c.n_calib):
        s_sym_t = pdq.calibrate_static_sym(torch.from_numpy(c.calib(b)).to(torch.bfloat16).cuda(), mm_sym,
                                           finalize=b == c.n_calib - 1)
    s_sym = float(s_sym_t.item())
    # and the 254-level zero-point grid's (S, Z)
    mm_zp = pdq.minmax_state("cuda")
    for b in range(c.n_calib):
        zp_out = pdq.calibrate_zeropoint(torch.from_numpy(c.calib(b)).to(torch.bfloat16).cuda(), mm_zp,
                                         finalize=b == c.n_calib - 1)
    s_zp, z_zp = float(zp_out[0].item()), int(zp_out[1].item())
    wq0, ws, cs = pdq.quantize_weight(torch.from_numpy(c.w()).to(torch.bfloat16).cuda())
    nrot = 64  # 64 x 16.8 MB = 1.07 GB of INT8 weights
    wqs = [wq0] + [wq0.clone() for _ in range(nrot - 1)]
    stream = torch.cuda.current_stream()
    res = {}
    gpu_out = {}  # host copies of each batch's first call, for the CPU-baseline leg's parity check
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    for m in c.batches:
        x = torch.from_numpy(c.x(m)).to(torch.bfloat16).cuda()
        xq = torch.empty(pdq.act_bytes(m, K), dtype=torch.int8, device="cuda")  # packed codes
        y = torch.empty((m, N), dtype=torch.bfloat16, device="cuda")
        sat.zero_()
        first = pdq.linear_decode(x, s, z, wq0, ws, cs, sat_count=sat, out=y, xq=xq, want_acc=True)
        torch.cuda.synchronize()
        nsat = int(sat.item())
        gpu_out[str(m)] = dict(xq=pdq.Codes(xq, m, K).unpack(), acc=first["acc"].cpu().numpy(),
                               y=y.cpu().view(torch.int16).numpy().view(np.uint16), sat=nsat)
        del first

        def call(i):
            pdq._call("pdq_linear_decode", pdq._p(x), pdq.BF16, m, K, K, s, z, pdq._p(wqs[i % nrot]),
                      pdq._p(ws), pdq._p(cs), None, N, pdq._p(xq), pdq._p(y), N, None, None,
                      pdq._stream(x.device))

        def gemv(i):
            pdq._call("pdq_gemm_static", pdq._p(xq), m, K, s, z, pdq._p(wqs[i % nrot]), pdq._p(ws),
                      pdq._p(cs), None, N, pdq._p(y), N, None, pdq._stream(x.device))

        iters = max(args.steps * 10, 200)
        settle(call, stream)
        ms_call = timed(call, iters, args.warmup * 4, stream)
        ms_gemv = timed(gemv, iters, args.warmup * 4, stream)
        # the same calls replayed from a HIP graph (one call per weight copy)
        # (all copies hold the same weights, so every replay must leave the
        # eager output in y)
        y_eager = y.clone()
        ms_call_g = graph_timed(call, nrot, max(args.steps // 2, 10), stream)
        if not torch.equal(y, y_eager):
            raise RuntimeError(f"decode M={m}: the replayed call changed the output")
        ms_gemv_g = graph_timed(gemv, nrot, max(args.steps // 2, 10), stream)
        if not torch.equal(y, y_eager):
            raise RuntimeError(f"decode M={m}: the replayed GEMV changed the output")

        def call_sym(i):
            pdq._call("pdq_linear_static_sym", pdq._p(x), pdq.BF16, m, K, K, s_sym, pdq._p(wqs[i % nrot]),
                      pdq._p(ws), None, N, pdq._p(xq), pdq._p(y), N, None, None, pdq._stream(x.device))

        ms_sym_g = graph_timed(call_sym, nrot, max(args.steps // 2, 10), stream)

        def call_zp(i):
            pdq._call("pdq_linear_zeropoint", pdq._p(x), pdq.BF16, m, K, K, s_zp, z_zp, pdq._p(wqs[i % nrot]),
                      pdq._p(ws), pdq._p(cs), None, N, pdq._p(xq), pdq._p(y), N, None, None, pdq._stream(x.device))

        ms_zp_g = graph_timed(call_zp, nrot, max(args.steps // 2, 10), stream)
        # algorithmic bytes: int8 W once, bf16 X, bf16 Y, w_scale + colsum
        call_bytes = N * K + 2 * m * K + 2 * m * N + 8 * N
        gemv_bytes = N * K + m * K + 2 * m * N + 8 * N
        res[str(m)] = dict(us_call=ms_call * 1e3, us_gemv=ms_gemv * 1e3,
                           us_call_graph=ms_call_g * 1e3, us_gemv_graph=ms_gemv_g * 1e3,
                           call_GBps=call_bytes / (ms_call * 1e-3) / 1e9,
                           gemv_GBps=gemv_bytes / (ms_gemv * 1e-3) / 1e9,
                           call_graph_GBps=call_bytes / (ms_call_g * 1e-3) / 1e9,
                           gemv_graph_GBps=gemv_bytes / (ms_gemv_g * 1e-3) / 1e9,
                           gemv_graph_frac=gemv_bytes / (ms_gemv_g * 1e-3) / 1e9 / PEAK_HBM_GBS,
                           gemv_frac=gemv_bytes / (ms_gemv * 1e-3) / 1e9 / PEAK_HBM_GBS,
                           saturated=nsat, saturated_frac=nsat / (m * K),
                           us_call_static_sym_graph=ms_sym_g * 1e3, us_call_zeropoint_graph=ms_zp_g * 1e3)
    # the C_s / C_g pair at a few M, over 16 of the weight copies (the --sweep
    # protocol; the full sweep over M = 1 .. 8192 is `bench.py --sweep`)
    x_all = torch.from_numpy(c.x(max(SWEEP_M))).to(torch.bfloat16).cuda()
    cs_cg = {str(m): cs_cg_point(torch, pdq, m, x_all, s, z, wqs, ws, cs, 16, 10 if m <= 256 else 4)
             for m in CS_CG_M}
    del wqs, x_all
    return dict(S=s, Z=z, S_sym=s_sym, S_zp=s_zp, Z_zp=z_zp, K=K, N=N, per_batch=res, cs_cg=cs_cg,
                gpu_out=gpu_out)


DECODE_SWEEP_N = (4096, 16384, 65536, 131072)  # K = 4096: 16.8 .. 537 MB of INT8 weight


def bench_decode_weights(args, torch, pdq, synth, s, z):
    """The static decode linear at M = 1 (the one-launch call, and the GEMV on
    its codes) for INT8 weights of 16.8 to 537 MB (K = 4096, N = 4096 ..
    131072), with the calibrated S and Z of the decode workload: HIP-graph
    replays over weight copies rotated through at least 1 GB, so that every
    call streams its weight from HBM.  Weights N(0, 0.02) drawn on the device
    from a seeded generator (the host generator would take seconds at this
    size); the activation row is the decode recipe's."""
    c = synth.Decode()
    K = c.K
    x = torch.from_numpy(c.x(1)).to(torch.bfloat16).cuda()
    xq = torch.empty(pdq.act_bytes(1, K), dtype=torch.int8, device="cuda")
    pdq.quantize_static(x, s, z, xq=xq)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(901)
    stream = torch.cuda.current_stream()
    res = {}
    for n in DECODE_SWEEP_N:
        w = (torch.randn((n, K), device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
        wq0, ws, cs = pdq.quantize_weight(w)
        del w
        copies = max(2, -(-(1 << 30) // wq0.numel()))
        wqs = [wq0] + [wq0.clone() for _ in range(copies - 1)]
        y = torch.empty((1, n), dtype=torch.bfloat16, device="cuda")

        def call(i):
            pdq._call("pdq_linear_decode", pdq._p(x), pdq.BF16, 1, K, K, s, z, pdq._p(wqs[i % copies]),
                      pdq._p(ws), pdq._p(cs), None, n, pdq._p(xq), pdq._p(y), n, None, None, pdq._stream(x.device))

        def gemv(i):
            pdq._call("pdq_gemm_static", pdq._p(xq), 1, K, s, z, pdq._p(wqs[i % copies]), pdq._p(ws), pdq._p(cs),
                      None, n, pdq._p(y), n, None, pdq._stream(x.device))

        replays = max(10, 256 // copies)
        settle(call, stream)
        ms_call = graph_timed(call, copies, replays, stream)
        ms_gemv = graph_timed(gemv, copies, replays, stream)
        call_bytes = n * K + 2 * K + 2 * n + 8 * n
        gemv_bytes = n * K + K + 2 * n + 8 * n
        res[str(n)] = dict(weight_MB=round(n * K / 1e6, 1), copies=copies,
                           us_call=round(ms_call * 1e3, 2),
                           call_GBps=round(call_bytes / (ms_call * 1e-3) / 1e9, 1),
                           call_frac=round(call_bytes / (ms_call * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                           us_gemv=round(ms_gemv * 1e3, 2),
                           gemv_GBps=round(gemv_bytes / (ms_gemv * 1e-3) / 1e9, 1),
                           gemv_frac=round(gemv_bytes / (ms_gemv * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
        del wqs, wq0, ws, cs, y
        torch.cuda.empty_cache()
    return res


SWEEP_M = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192)


CS_CG_M = (1, 64, 512, 4096)  # the compact C_s / C_g figures of the default run


def cs_cg_point(torch, pdq, m, x_all, s, z, wqs, ws, cs, nrot, replays):
    """C_s and C_g of one M on the decode linear: per-token dynamic
    (quantize_per_token + gemm_per_token) and per-tensor static
    (quantize_static + gemm_static, and the one-launch decode call where it
    applies), each from HIP-graph replays of nrot calls over the rotated
    weight copies."""
    K, N = x_all.shape[1], ws.shape[0]
    x = x_all[:m]
    xq = torch.empty(pdq.act_bytes(m, K), dtype=torch.int8, device="cuda")  # packed codes
    xsc = torch.empty(m, dtype=torch.float32, device="cuda")
    y = torch.empty((m, N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def dq(i):
        pdq._call("pdq_quantize_per_token", pdq._p(x), pdq.BF16, m, K, K, pdq._p(xq), pdq._p(xsc), pdq._stream(x.device))

    def dg(i):
        pdq._call("pdq_gemm_per_token", pdq._p(xq), pdq._p(xsc), m, K, pdq._p(wqs[i % nrot]), pdq._p(ws),
                  None, N, pdq._p(y), N, None, pdq._stream(x.device))

    def sq(i):
        pdq._call("pdq_quantize_static", pdq._p(x), pdq.BF16, m, K, K, s, z, pdq._p(xq), None, pdq._stream(x.device))

    def sg(i):
        pdq._call("pdq_gemm_static", pdq._p(xq), m, K, s, z, pdq._p(wqs[i % nrot]), pdq._p(ws), pdq._p(cs),
                  None, N, pdq._p(y), N, None, pdq._stream(x.device))

    def call(i):
        pdq._call("pdq_linear_decode", pdq._p(x), pdq.BF16, m, K, K, s, z, pdq._p(wqs[i % nrot]),
                  pdq._p(ws), pdq._p(cs), None, N, pdq._p(xq), pdq._p(y), N, None, None, pdq._stream(x.device))

    dq(0)
    settle(dg, stream, 50.0)
    t = {name: graph_timed(fn, nrot, replays, stream) * 1e3
         for name, fn in (("dyn_quant", dq), ("dyn_gemm", dg), ("static_quant", sq),
                          ("static_gemm", sg), ("static_call", call))}
    t["dyn_total"] = t["dyn_quant"] + t["dyn_gemm"]
    t["static_total"] = t["static_quant"] + t["static_gemm"]
    t["dyn_Cs_over_Cg"] = t["dyn_quant"] / t["dyn_gemm"]
    t["static_Cs_over_Cg"] = t["static_quant"] / t["static_gemm"]
    t["gemm_TOPS_dyn"] = 2.0 * m * N * K / (t["dyn_gemm"] * 1e-6) / 1e12
    return {k: round(v, 3) for k, v in t.items()}


def bench_sweep(args, torch, pdq, synth):
    """C_s / C_g of the two activation schemes over M on the decode linear 4096 -> 4096:
    per-token dynamic (quantize_per_token + gemm_per_token) against per-tensor
    static (quantize_static + gemm_static, and the one-launch decode call where
    it applies), every figure from HIP-graph replays over 16 weight copies (269
    MB, more than the MALL).  The quantization cost C_s and the GEMM cost C_g
    are the two terms the pages weigh when they keep dynamic quantization for
    prefill and static for decode."""
    c = synth.Decode()
    K, N = c.K, c.N
    log(f"[sweep] calibrating on {c.n_calib} batches of [{c.calib_tokens},{K}]")
    mm = pdq.minmax_state("cuda")
    for b in range(c.n_calib):
        out = pdq.calibrate_static(torch.from_numpy(c.calib(b)).to(torch.bfloat16).cuda(), mm,
                                   finalize=b == c.n_calib - 1)
    s, z = float(out[0].item()), int(out[1].item())
    wq0, ws, cs = pdq.quantize_weight(torch.from_numpy(c.w()).to(torch.bfloat16).cuda())
    nrot = 16
    wqs = [wq0] + [wq0.clone() for _ in range(nrot - 1)]
    x_all = torch.from_numpy(c.x(max(SWEEP_M))).to(torch.bfloat16).cuda()
    rows = {}
    for m in SWEEP_M:
        t = cs_cg_point(torch, pdq, m, x_all, s, z, wqs, ws, cs, nrot, 20 if m <= 256 else 4)
        rows[str(m)] = t
        log(f"[sweep] M={m:5d}: dynamic {t['dyn_quant']:8.2f} + {t['dyn_gemm']:8.2f} us, static "
            f"{t['static_quant']:8.2f} + {t['static_gemm']:8.2f} us (one call {t['static_call']:8.2f} us)")
    del wqs
    return dict(S=s, Z=z, K=K, N=N, per_m=rows)


def bench_silu_mul(args, torch, pdq, synth):
    """The down projection's input of the decoder block: h = SiLU(gate) * up over
    8192 tokens x 14336, quantized per token by the fused kernel (gate and up
    read once, codes written, h never stored), against the same result formed
    unfused (torch's SiLU and multiply writing bf16 h, then the library's
    per-token quantizer reading it back), and the whole down projection
    (fused quantizer + INT8 GEMM 14336 -> 4096)."""
    c = synth.DecoderBlock()
    g, u = c.down_gate_up()
    M, K = g.shape
    gu = torch.from_numpy(np.concatenate([g, u], axis=1)).to(torch.bfloat16).cuda()  # [M, 2K]
    del g, u
    gate, up = gu[:, :K], gu[:, K:]
    _, n_down, _ = c.linears[3]
    wq, ws, _ = pdq.quantize_weight(torch.from_numpy(c.w(3)).to(torch.bfloat16).cuda())
    xq = pdq.Codes.empty(M, K, "cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")
    y = torch.empty((M, n_down), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    dv = pdq._stream(gu.device)

    def fused(i):
        pdq._call("pdq_silu_mul_quantize_per_token", pdq._p(gate), pdq._p(up), pdq.BF16, M, K, 2 * K, 2 * K,
                  pdq._p(xq), pdq._p(xs), None, 0, dv)

    def unfused(i):
        h = torch.nn.functional.silu(gate) * up
        pdq._call("pdq_quantize_per_token", pdq._p(h), pdq.BF16, M, K, K, pdq._p(xq), pdq._p(xs), dv)

    def linear(i):
        pdq._call("pdq_linear_prefill_silu_mul", pdq._p(gate), pdq._p(up), pdq.BF16, M, K, 2 * K, 2 * K,
                  pdq._p(wq), pdq._p(ws), None, n_down, pdq._p(xq), pdq._p(xs), pdq._p(y), n_down, None, dv)

    settle(fused, stream)
    ms_fused = timed(fused, 20, 5, stream)
    ms_unfused = timed(unfused, 10, 3, stream)
    ms_linear = timed(linear, 10, 3, stream)
    nbytes = 2 * M * K * 2 + M * K + 4 * M
    return dict(M=M, K=K, N=n_down, ms_fused=ms_fused, ms_unfused=ms_unfused, ms_linear=ms_linear,
                bytes=nbytes, ops=2.0 * M * n_down * K)


TILE_SWEEP_N = (8192, 9216, 10240, 11008, 12288)


def bench_tile_sweep(args, torch, pdq, synth):
    """The prefill INT8 GEMM (M = K = 4096, the prefill workload's codes) at several
    N: 512 .. 768 tiles of 256 x 256, i.e. 2 .. 3 rounds of one tile per CU on the
    256 CUs.  Each N is timed with HIP events over 60 launches rotating 4 weight
    copies, once with N rising and once with N falling (the clock drifts with the
    board's thermal state)."""
    c = synth.Prefill7B()
    M, K = c.M, c.K
    x = torch.from_numpy(c.x()).to(torch.bfloat16).cuda()
    w_host = torch.from_numpy(c.w()).to(torch.bfloat16)
    nmax = max(TILE_SWEEP_N)
    reps = -(-nmax // w_host.shape[0])
    w_all = torch.cat([w_host] * reps, 0)[:nmax].cuda()  # rows repeat: same distribution
    xq = torch.empty(pdq.act_bytes(M, K), dtype=torch.int8, device="cuda")
    xsc = torch.empty(M, dtype=torch.float32, device="cuda")
    pdq.quantize_per_token(x, xq=xq, x_scale=xsc)
    xqs = [xq] + [xq.clone() for _ in range(3)]
    stream = torch.cuda.current_stream()
    weights = {}
    for n in TILE_SWEEP_N:
        wq0, wsc, _ = pdq.quantize_weight(w_all[:n].contiguous())
        weights[n] = ([wq0] + [wq0.clone() for _ in range(3)], wsc)
    rows = {}
    for direction, order in (("up", TILE_SWEEP_N), ("down", TILE_SWEEP_N[::-1])):
        for n in order:
            wqs, wsc = weights[n]
            y = torch.empty((M, n), dtype=torch.bfloat16, device="cuda")

            def gemm(i):
                r = i % 4
                pdq._call("pdq_gemm_per_token", pdq._p(xqs[r]), pdq._p(xsc), M, K, pdq._p(wqs[r]),
                          pdq._p(wsc), None, n, pdq._p(y), n, None, pdq._stream(x.device))

            us = timed(gemm, 60, 10, stream) * 1e3
            tiles = -(-M // 256) * -(-n // 256)
            r = rows.setdefault(str(n), {"tiles": tiles, "rounds": round(tiles / 256, 4)})
            r["us_" + direction] = round(us, 2)
            r["TOPS_" + direction] = round(2.0 * M * n * K / (us * 1e-6) / 1e12, 1)
            log(f"[tile sweep] N={n} ({tiles} tiles, {tiles / 256:.3f} rounds) {direction}: {us:.1f} us")
    return dict(M=M, K=K, per_n=rows)


def bench_block(args, torch, pdq, synth):
    """The decoder-block linear set (QKV 4096->12288, O 4096->4096, gate+up
    4096->28672, down 14336->4096), one shared INT8 weight copy per linear:
    a prefill pass over 8192 tokens (per-token dynamic) and decode steps at
    batch 32 (per-tensor static, calibrated on 50 batches of 512 tokens per
    linear), weights rotated over 4 copies of the set (~1 GB)."""
    c = synth.DecoderBlock()
    nrot = 4
    lin = []
    for l, (name, n, k) in enumerate(c.linears):
        wq, ws, cs = pdq.quantize_weight(torch.from_numpy(c.w(l)).to(torch.bfloat16).cuda())
        mm = pdq.minmax_state("cuda")
        for b in range(50):
            out = pdq.calibrate_static(torch.from_numpy(c.calib(l, b)).to(torch.bfloat16).cuda(), mm,
                                       finalize=b == 49)
        s, z = float(out[0].item()), int(out[1].item())
        lin.append(dict(name=name, n=n, k=k, wqs=[wq] + [wq.clone() for _ in range(nrot - 1)], ws=ws, cs=cs,
                        s=s, z=z))
        log(f"[block] {name} {n}x{k}: S={s:.5f} Z={z}")
    stream = torch.cuda.current_stream()
    # prefill: the four linears on 8192 tokens each
    M = c.prefill_tokens
    for l, d in enumerate(lin):
        d["x"] = torch.from_numpy(c.prefill_x(l)).to(torch.bfloat16).cuda()
        d["xq"] = torch.empty(pdq.act_bytes(M, d["k"]), dtype=torch.int8, device="cuda")
        d["xs"] = torch.empty(M, dtype=torch.float32, device="cuda")
        d["y"] = torch.empty((M, d["n"]), dtype=torch.bfloat16, device="cuda")

    def prefill(i):
        for d in lin:
            pdq._call("pdq_linear_prefill", pdq._p(d["x"]), pdq.BF16, M, d["k"], d["k"], pdq._p(d["wqs"][i % nrot]),
                      pdq._p(d["ws"]), None, d["n"], pdq._p(d["xq"]), pdq._p(d["xs"]), pdq._p(d["y"]), d["n"], None,
                      pdq._stream(d["x"].device))

    settle(prefill, stream)
    ms_prefill = timed(prefill, max(args.steps // 5, 5), max(args.warmup // 10, 3), stream)
    ops = sum(2.0 * M * d["n"] * d["k"] for d in lin)
    for d in lin:
        del d["x"], d["xq"], d["xs"], d["y"]
    # decode: 256 steps at batch 32, each step the four linears on its own inputs
    B, T = c.decode_batch, c.decode_steps
    for l, d in enumerate(lin):
        d["xt"] = torch.from_numpy(np.stack([c.decode_x(l, t) for t in range(T)])).to(torch.bfloat16).cuda()
        d["xq"] = torch.empty(pdq.act_bytes(B, d["k"]), dtype=torch.int8, device="cuda")
        d["y"] = torch.empty((B, d["n"]), dtype=torch.bfloat16, device="cuda")

    def step(t):
        for d in lin:
            x = d["xt"][t]
            pdq._call("pdq_linear_decode", pdq._p(x), pdq.BF16, B, d["k"], d["k"], d["s"], d["z"],
                      pdq._p(d["wqs"][t % nrot]), pdq._p(d["ws"]), pdq._p(d["cs"]), None, d["n"], pdq._p(d["xq"]),
                      pdq._p(d["y"]), d["n"], None, None, pdq._stream(x.device))

    settle(lambda i: step(i % T), stream)
    ms_step = graph_timed(step, T, 2, stream)
    wbytes = sum(d["n"] * d["k"] for d in lin)
    step_bytes = sum(d["n"] * d["k"] + 2 * B * d["k"] + 2 * B * d["n"] + 8 * d["n"] for d in lin)
    del lin
    return dict(ms_prefill=ms_prefill, prefill_ops=ops, ms_step=ms_step, weight_bytes=wbytes,
                step_bytes=step_bytes, steps=T, batch=B, tokens=M)


def bench_llm_int8(args, torch, pdq, synth):
    c = synth.LlmInt8()
    M, K, N = c.M, c.K, c.N
    log(f"[llm.int8] generating X[{M},{K}] and W[{N},{K}] ({c.dtype})")
    x_host, w_host = c.x(), c.w()
    x = torch.from_numpy(x_host).half().cuda()
    w16 = torch.from_numpy(w_host).half().cuda()
    wq0, ws, _ = pdq.quantize_weight(w16)
    nrot = 2
    wqs = [wq0] + [wq0.clone() for _ in range(nrot - 1)]
    max_out = 64
    ws_bytes = pdq.int8_outlier_workspace_bytes(M, N, K, max_out)
    work = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    xq = torch.empty(pdq.act_bytes(M, K), dtype=torch.int8, device="cuda")  # packed codes
    xs = torch.empty(M, dtype=torch.float32, device="cuda")
    idx = torch.empty(max_out, dtype=torch.int32, device="cuda")
    cnt = torch.empty(1, dtype=torch.int32, device="cuda")
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()

    def call(i):
        pdq._call("pdq_linear_int8_outlier", pdq._p(x), pdq.F16, M, K, K, c.threshold,
                  pdq._p(wqs[i % nrot]), pdq._p(ws), pdq._p(w16), K, None, N, pdq._p(y), N, pdq._p(xq),
                  pdq._p(xs), pdq._p(idx), pdq._p(cnt), max_out, pdq._p(work), ws_bytes, None,
                  pdq._stream(x.device))

    settle(call, stream)
    ms = timed(call, args.steps, args.warmup, stream)
    n_out = int(cnt.item())
    ops = 2.0 * M * N * K
    # one untimed call with the INT32 accumulators: its outputs, on the host,
    # for the CPU-baseline leg to compare with the oracle's same layer
    chk = pdq.linear_int8_outlier(x, c.threshold, wq0, ws, w16, max_outliers=max_out, want_acc=True,
                                  workspace=work)
    torch.cuda.synchronize()
    n_chk = int(chk["count"].item())
    gpu_out = dict(idx=chk["idx"][:min(n_chk, max_out)].cpu().numpy(), count=n_chk, xq=chk["xq"].unpack(),
                   x_scale=chk["x_scale"].cpu().numpy(), acc=chk["acc"].cpu().numpy(),
                   y=chk["y"].cpu().view(torch.int16).numpy().view(np.uint16))
    del chk
    return dict(M=M, K=K, N=N, ms=ms, n_outlier=n_out, int8_tops=ops / (ms * 1e-3) / 1e12,
                host=(x_host, w_host, c.threshold, gpu_out),
                side_flops=2.0 * M * N * n_out)


def run_env(torch) -> dict:
    """Versions and device of the run: PyTorch and its HIP runtime, the GPU's
    name, architecture and compute units, the library's build (hash of its
    kernel sources)."""
    props = torch.cuda.get_device_properties(0)
    env = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None), "device": props.name,
           "arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count,
           "memory_GB": round(props.total_memory / 1e9, 1)}
    try:
        import glob

        h = hashlib.sha256()
        for f in sorted(glob.glob(os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                               "w8a8_int8_quantized_absmax_amd", "csrc", "*"))):
            with open(f, "rb") as fh:
                h.update(fh.read())
        env["kernel_sources_sha256"] = h.hexdigest()[:16]
    except OSError:
        pass
    return env


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _parity(O, g, ref):
    """The GPU's outputs of one call (host copies) against the oracle's result
    for the same inputs: mismatch counts of the codes, scales, accumulators,
    saturation count and bf16 bits, and the bf16 output's error against the
    oracle's binary32 dequant (max relative error with the denominator floored
    at 1e-3 max|y|; mean absolute error against that value rounded to bf16)."""
    y32 = ref["y32"].astype(np.float64)
    ref_bits = O.to_bf16_bits(ref["y32"])
    got = O.bf16_bits_to_f32(g["y"]).astype(np.float64)
    floor = 1e-3 * max(float(np.abs(y32).max()), 1e-30)
    rel = float((np.abs(got - y32) / np.maximum(np.abs(y32), floor)).max())
    mae = float(np.mean(np.abs(got - O.bf16_bits_to_f32(ref_bits).astype(np.float64))))
    out = {"outputs": int(y32.size),
           "code_mismatches": int(np.count_nonzero(g["xq"] != ref["xq"])),
           "acc_mismatches": int(np.count_nonzero(g["acc"] != ref["acc"])),
           "y_bits_mismatches": int(np.count_nonzero(g["y"] != ref_bits)),
           "y_max_rel_err": rel, "y_mae": mae}
    if "x_scale" in g:
        out["scale_mismatches"] = int(np.count_nonzero(g["x_scale"].view(np.uint32) !=
                                                       ref["x_scale"].view(np.uint32)))
    if "sat" in g:
        out["saturation_count_equal"] = bool(g["sat"] == ref["sat"])
    return out


def _parity_llm_int8(O, g, ref):
    """The GPU's LLM.int8() outputs against the oracle's: the outlier columns,
    codes, scales and INT32 accumulators exactly; the f16 output (whose
    16-bit side product the oracle sums in binary64) by its max relative error
    (denominator floored at 1e-3 max|y|) and its MAE against the oracle's
    binary64 value rounded to f16."""
    y64 = ref["y64"]
    got = g["y"].view(np.float16).astype(np.float64)
    floor = 1e-3 * max(float(np.abs(y64).max()), 1e-30)
    rel = float((np.abs(got - y64) / np.maximum(np.abs(y64), floor)).max())
    mae = float(np.mean(np.abs(got - O.to_f16(y64).astype(np.float64))))
    return {"outputs": int(y64.size), "outlier_columns_equal": bool(g["count"] == len(ref["cols"]) and
                                                                    np.array_equal(g["idx"], ref["cols"])),
            "code_mismatches": int(np.count_nonzero(g["xq"] != ref["xq"])),
            "scale_mismatches": int(np.count_nonzero(g["x_scale"].view(np.uint32) != ref["x_scale"].view(np.uint32))),
            "acc_mismatches": int(np.count_nonzero(g["acc"] != ref["acc"])),
            "y_max_rel_err": rel, "y_mae": mae}


def cpu_baseline(pre, synth, llm_host=None, dec=None):
    """The oracle (plain numpy, binary64 BLAS for the exact integer products)
    timed on this host's cores: whole prefill linears (the headline workload,
    `value`), the same linear stage by stage, the offline steps, the decode
    linear at M = 1, 8, 32, 64 (GB/s over the same algorithmic bytes as the
    GPU figures), the LLM.int8() layer (TOPS of its INT8 product), and the tiny
    and M = 1 decode workloads on one thread.  About 20 s of host time."""
    import oracle.pdq_oracle as O

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threadpool_limits, blas_threads = None, os.cpu_count() or 1
    cores = len(os.sched_getaffinity(0))
    clock = time.perf_counter
    out = {"unit": "TOPS", "kind": "oracle", "cores": cores, "blas_threads": int(blas_threads),
           "cpu_model": _cpu_model()}
    x, w = pre["x_host"], pre["w_host"]
    M, K, N = pre["M"], pre["K"], pre["N"]
    t0 = clock()
    wq, sw, _ = O.quantize_weight(w)
    t_wq = clock() - t0
    # whole prefill linears, repeated until about 6 s (at least 2 runs)
    runs, t0 = 0, clock()
    while True:
        ref = O.linear_prefill(x, wq, sw)
        runs += 1
        dt = clock() - t0
        if (dt >= 6.0 and runs >= 2) or runs >= 30:
            break
    out["value"] = pre["ops"] * runs / dt / 1e12
    parity = {}
    if pre.get("gpu_out") is not None:
        parity["prefill"] = _parity(O, pre["gpu_out"], ref)
    del ref
    out["sample"] = (f"{runs} full prefill linears {M}x{K}->{N} (per-token quant, exact integer GEMM via a "
                     f"binary64 BLAS product, binary32 epilogue) in {dt:.1f} s")
    # the same linear stage by stage
    t0 = clock()
    xq, sx = O.quantize_rows_absmax(x)
    t_q = clock() - t0
    t0 = clock()
    acc = O.int_matmul(xq, wq)
    t_g = clock() - t0
    t0 = clock()
    O.dequantize(acc, sx, sw)
    t_e = clock() - t0
    del acc
    out["prefill_stages_s"] = {"quantize_per_token": round(t_q, 4), "int_gemm": round(t_g, 4),
                               "dequant_epilogue": round(t_e, 4), "weight_quant_offline": round(t_wq, 4)}
    out["prefill_quant_GBps"] = round((2 * M * K + M * K + 4 * M) / t_q / 1e9, 3)
    out["prefill_gemm_TOPS"] = round(pre["ops"] / t_g / 1e12, 4)
    # decode linear 4096 -> 4096 with the calibrated static (S, Z)
    c = synth.Decode()
    wd = c.w()
    wqd, swd, csd = O.quantize_weight(wd)
    cal = [c.calib(b) for b in range(10)]
    t0 = clock()
    state = None
    for xb in cal:
        state = O.minmax_update(state, xb)
    O.minmax_finalize(state)
    out["calibration_s_per_batch"] = round((clock() - t0) / len(cal), 5)
    s_dec, z_dec = (dec["S"], dec["Z"]) if dec else O.calibrate(cal)[1:]
    dec_out = {}
    for m in c.batches:
        xm = c.x(m)
        reps, t0 = 0, clock()
        while True:
            dref = O.linear_decode(xm, np.float32(s_dec), z_dec, wqd, swd, csd)
            reps += 1
            if clock() - t0 >= 0.5 and reps >= 3:
                break
        us = (clock() - t0) / reps * 1e6
        nbytes = c.N * c.K + 2 * m * c.K + 2 * m * c.N + 8 * c.N
        dec_out[str(m)] = {"us_call": round(us, 1), "GBps": round(nbytes / (us * 1e-6) / 1e9, 3)}
        g = (dec or {}).get("gpu_out", {}).get(str(m))
        if g is not None:
            parity.setdefault("decode", {})[str(m)] = _parity(O, g, dref)
    out["decode"] = dec_out
    # the LLM.int8() layer: outlier detection, then the whole decomposition
    if llm_host is not None:
        x8, w8, thr, g8 = llm_host
        wq8, sw8, _ = O.quantize_weight(w8)
        t0 = clock()
        O.outlier_columns(x8, thr)
        t_det = clock() - t0
        t0 = clock()
        ref8 = O.linear_int8_outlier(x8, w8, wq8, sw8, thr)
        t_l = clock() - t0
        if g8 is not None:
            parity["llm_int8"] = _parity_llm_int8(O, g8, ref8)
        del ref8
        ops8 = 2.0 * x8.shape[0] * w8.shape[0] * x8.shape[1]
        out["llm_int8"] = {"s": round(t_l, 3), "int8_TOPS": round(ops8 / t_l / 1e12, 4),
                           "outlier_detection_s": round(t_det, 4)}
    # one thread: the tiny workload's prefill and decode, and the M = 1 decode linear
    if threadpool_limits is not None:
        tiny = synth.Tiny()
        xt, wt = tiny.x(), tiny.w()
        with threadpool_limits(1):
            rq, rs, rc = O.quantize_weight(wt)
            t0 = clock()
            for _ in range(20):
                O.linear_prefill(xt, rq, rs)
            t_tp = (clock() - t0) / 20
            t0 = clock()
            for _ in range(20):
                O.linear_decode(xt, np.float32(0.5), 3, rq, rs, rc)
            t_td = (clock() - t0) / 20
            x1 = c.x(1)
            t0 = clock()
            for _ in range(3):
                O.linear_decode(x1, np.float32(s_dec), z_dec, wqd, swd, csd)
            t_d1 = (clock() - t0) / 3
        out["one_thread"] = {"tiny_prefill_us": round(t_tp * 1e6, 1), "tiny_decode_us": round(t_td * 1e6, 1),
                             "decode_m1_us": round(t_d1 * 1e6, 1),
                             "decode_m1_GBps": round((c.N * c.K + 2 * c.K + 2 * c.N + 8 * c.N) / t_d1 / 1e9, 3)}
    if parity:
        out["parity"] = parity
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "silu", "block", "block-gemv"], default="all",
                    help="prefill: the headline line without the other workloads; decode: only the decode "
                         "measurements, in a line of their own (for counter collection); silu: only the "
                         "fused SiLU*up quantizer and its down projection; block-gemv: the decoder block's "
                         "four decode GEMMs at batch 32, six calls each (for counter collection)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline run: the per-token vs static C_s / C_g sweep over "
                         "M on the decode linear (one JSON line of its own)")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="instead of the headline run: the prefill INT8 GEMM at N = 8192 .. 12288 "
                         "(2 .. 3 rounds of 256 x 256 tiles on 256 CUs), one JSON line of its own")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="also run a fill and a plain device copy of this many MiB (known HBM "
                         "traffic, for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from w8a8_int8_quantized_absmax_amd import pdq, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    pdq.lib()
    if args.sweep:
        sw = bench_sweep(args, torch, pdq, synth)
        print(json.dumps({"metric": "cs_cg_sweep_us", "unit": "us", "n_gpus": 1, "data": "synthetic",
                          "config": {"workload": "decode linear 4096 -> 4096, bf16 activations, "
                                                 "per-token dynamic vs per-tensor static INT8",
                                     "M": list(SWEEP_M)},
                          "S": sw["S"], "Z": sw["Z"], "per_m": sw["per_m"]}), flush=True)
        return
    if args.tile_sweep:
        ts = bench_tile_sweep(args, torch, pdq, synth)
        print(json.dumps({"metric": "gemm_us_vs_tiles", "unit": "us", "n_gpus": 1, "data": "synthetic",
                          "config": {"workload": "prefill INT8 GEMM 4096 x 4096 -> N, per-token codes",
                                     "M": ts["M"], "K": ts["K"], "N": list(TILE_SWEEP_N)},
                          "per_n": ts["per_n"]}), flush=True)
        return
    if args.copy_probe:
        # known traffic: the fill kernel writes size bytes, the copy kernel
        # reads size bytes and writes size bytes (far more than the 256 MB MALL)
        n = args.copy_probe * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda")
        a.fill_(1.0)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.only == "silu":
        smq = bench_silu_mul(args, torch, pdq, synth)
        print(json.dumps({"metric": "fused SiLU*up + per-token INT8 GB/s", "unit": "GB/s", "n_gpus": 1,
                          "data": "synthetic", "config": {"workload": "decoder block down-projection input "
                                                                      "8192 x 14336 bf16"},
                          "fused_us": round(smq["ms_fused"] * 1e3, 2),
                          "fused_GBps": round(smq["bytes"] / (smq["ms_fused"] * 1e-3) / 1e9, 1),
                          "unfused_us": round(smq["ms_unfused"] * 1e3, 2),
                          "down_projection_us": round(smq["ms_linear"] * 1e3, 1)}), flush=True)
        return
    if args.only == "block":
        blk = bench_block(args, torch, pdq, synth)
        print(json.dumps({"metric": "decoder block decode step GB/s", "unit": "GB/s", "n_gpus": 1,
                          "data": "synthetic",
                          "config": {"workload": "QKV 4096->12288, O 4096->4096, gate+up 4096->28672, "
                                                 "down 14336->4096; prefill 8192 tokens, decode batch 32"},
                          "prefill_us": round(blk["ms_prefill"] * 1e3, 1),
                          "decode_us_per_step": round(blk["ms_step"] * 1e3, 2),
                          "decode_GBps": round(blk["step_bytes"] / (blk["ms_step"] * 1e-3) / 1e9, 1)}), flush=True)
        return
    if args.only == "block-gemv":
        # random weights and activations of the decoder block's shapes, six
        # eager GEMM calls per linear in the block's order; the line reports
        # the kernel plan (the timings of this workload are the block's)
        c = synth.DecoderBlock()
        out = {}
        for name, n, k in c.linears:
            wq, ws, cs = pdq.quantize_weight((torch.randn(n, k, device="cuda") * 0.02).to(torch.bfloat16))
            xq = pdq.quantize_static((torch.randn(c.decode_batch, k, device="cuda") + 0.1).to(torch.bfloat16),
                                     0.05, 3)
            for _ in range(6):
                pdq.gemm_static(xq, 0.05, 3, wq, ws, cs)
            torch.cuda.synchronize()
            out[name] = {"N": n, "K": k, "channels_per_workgroup": pdq.skinny_channels(c.decode_batch, n)}
            del wq, ws, cs, xq
        print(json.dumps({"metric": "decoder block decode GEMMs", "unit": "us", "n_gpus": 1, "data": "synthetic",
                          "config": {"workload": "static INT8 codes, batch 32"}, "per_linear": out}), flush=True)
        return
    if args.only == "decode":
        dec = bench_decode(args, torch, pdq, synth)
        print(json.dumps({"metric": "decode GB/s", "unit": "GB/s", "n_gpus": 1, "data": "synthetic",
                          "config": {"workload": "decode linear 4096 -> 4096, static per-tensor INT8"},
                          "decode": dec}), flush=True)
        return
    pre = bench_prefill(args, torch, pdq, synth)
    log(f"[prefill] step {pre['ms_step']*1e3:.1f} us (quant {pre['ms_quant']*1e3:.1f} us, "
        f"GEMM {pre['ms_gemm']*1e3:.1f} us = {pre['gemm_tops']:.0f} TOPS)")
    if pre["ms_lib"] is not None:
        log(f"[prefill] hipBLASLt INT8 GEMM (torch._int_mm, INT32 out) {pre['ms_lib']*1e3:.1f} us")
    log(f"[prefill asym] step {pre['ms_step_asym']*1e3:.1f} us (quant {pre['ms_quant_asym']*1e3:.1f} us, "
        f"GEMM {pre['ms_gemm_asym']*1e3:.1f} us)")
    dec = llm = blk = smq = dws = None
    if args.only == "all":
        dec = bench_decode(args, torch, pdq, synth)
        for m, r in dec["per_batch"].items():
            log(f"[decode] M={m}: call {r['us_call']:.2f} us, GEMV {r['us_gemv']:.2f} us = "
                f"{r['gemv_GBps']:.0f} GB/s; from a graph: call {r['us_call_graph']:.2f} us "
                f"({r['call_graph_GBps']:.0f} GB/s), GEMV {r['us_gemv_graph']:.2f} us "
                f"({r['gemv_graph_GBps']:.0f} GB/s); saturated {r['saturated']}; static symmetric call "
                f"{r['us_call_static_sym_graph']:.2f} us, zero-point call {r['us_call_zeropoint_graph']:.2f} us")
        dws = bench_decode_weights(args, torch, pdq, synth, dec["S"], dec["Z"])
        for n, r in dws.items():
            log(f"[decode M=1, 4096 -> {n}, {r['weight_MB']} MB] call {r['us_call']:.2f} us = "
                f"{r['call_GBps']:.0f} GB/s ({100 * r['call_frac']:.1f}%), GEMV {r['us_gemv']:.2f} us = "
                f"{r['gemv_GBps']:.0f} GB/s ({100 * r['gemv_frac']:.1f}%)")
        llm = bench_llm_int8(args, torch, pdq, synth)
        log(f"[llm.int8] {llm['ms']*1e3:.1f} us, {llm['int8_tops']:.0f} TOPS, |O|={llm['n_outlier']}")
        blk = bench_block(args, torch, pdq, synth)
        log(f"[block] prefill of 4 linears x {blk['tokens']} tokens {blk['ms_prefill']*1e3:.0f} us = "
            f"{blk['prefill_ops'] / (blk['ms_prefill'] * 1e-3) / 1e12:.0f} TOPS; decode step (4 linears, "
            f"batch {blk['batch']}) {blk['ms_step']*1e3:.1f} us = "
            f"{blk['step_bytes'] / (blk['ms_step'] * 1e-3) / 1e9:.0f} GB/s")
        smq = bench_silu_mul(args, torch, pdq, synth)
        log(f"[silu*up quant] fused {smq['ms_fused']*1e3:.1f} us = "
            f"{smq['bytes'] / (smq['ms_fused'] * 1e-3) / 1e9:.0f} GB/s; unfused (torch SiLU*up + quantizer) "
            f"{smq['ms_unfused']*1e3:.1f} us; down projection {smq['ms_linear']*1e3:.1f} us")

    value = pre["ops"] / (pre["ms_step"] * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "prefill linear, 4096 tokens x (4096 -> 11008), bf16 in/out, per-token "
                               "dynamic symmetric INT8 activations, per-channel INT8 weights",
                   "M": pre["M"], "K": pre["K"], "N": pre["N"], "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(pre["gemm_tops"], 2), "peak": PEAK_INT8_TOPS,
                     "unit": "TFLOP/s", "frac": round(pre["gemm_tops"] / PEAK_INT8_TOPS, 4),
                     "traffic": traffic_for(pre["gemm_bytes"]),
                     "kernel": "k_gemm_i8 (INT8 MFMA GEMM + bf16 epilogue)",
                     "us_per_launch": round(pre["ms_gemm"] * 1e3, 2),
                     "sclk_during_gemm": pre["sclk"]},
        "env": run_env(torch),
        "settle": {"ms_before_each_timed_region": SETTLE_MS,
                   "why": "the first ~35 ms of launches after the GPU has idled (input generation on the host) "
                          "run up to 30% slower while the clock ramps up; each timed region is preceded by "
                          "this much untimed work of its own kind, so it measures the steady state"},
        "cold_start": {"prefill_step_us": round(pre["ms_step_cold"] * 1e3, 2),
                       "TOPS": round(pre["ops"] / (pre["ms_step_cold"] * 1e-3) / 1e12, 1),
                       "what": f"the same {args.steps} steps after {args.warmup} warmups, timed right after "
                               "1.5 s of GPU idle, without the settling phase"},
        "prefill_quant": {"us": round(pre["ms_quant"] * 1e3, 2),
                          "GBps": round(pre["quant_bytes"] / (pre["ms_quant"] * 1e-3) / 1e9, 1)},
        "reference_library_gemm": None if pre["ms_lib"] is None else {
            "what": "hipBLASLt INT8 GEMM via torch._int_mm on the same codes, INT32 out, no quantization "
                    "or epilogue", "us": round(pre["ms_lib"] * 1e3, 2),
            "TOPS": round(pre["ops"] / (pre["ms_lib"] * 1e-3) / 1e12, 1)},
        "prefill_asym": {"us_step": round(pre["ms_step_asym"] * 1e3, 2),
                         "us_quant": round(pre["ms_quant_asym"] * 1e3, 2),
                         "us_gemm": round(pre["ms_gemm_asym"] * 1e3, 2),
                         "gemm_TOPS": round(pre["ops"] / (pre["ms_gemm_asym"] * 1e-3) / 1e12, 1),
                         "frac": round(pre["ops"] / (pre["ms_gemm_asym"] * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4)},
    }
    if dec:
        out["decode"] = {"unit": "GB/s", "peak": PEAK_HBM_GBS, "S": dec["S"], "Z": dec["Z"], "S_sym": dec["S_sym"],
                         "S_zeropoint": dec["S_zp"], "Z_zeropoint": dec["Z_zp"],
                         "per_batch": {m: {k: round(v, 5) if isinstance(v, float) else v
                                           for k, v in r.items()} for m, r in dec["per_batch"].items()}}
        if dws:
            out["decode_weight_sweep"] = {
                "workload": "static decode linear at M = 1, K = 4096, N = 4096 .. 131072 (16.8 .. 537 MB of INT8 "
                            "weight), HIP-graph replays over copies rotated through >= 1 GB; the one-launch call "
                            "and the GEMV on its codes",
                "unit": "GB/s", "peak": PEAK_HBM_GBS, "per_N": dws}
        out["cs_cg"] = {"workload": "decode linear 4096 -> 4096, bf16 activations: quantizer cost C_s and "
                                    "GEMM cost C_g (us, HIP-graph replays over 16 weight copies), per-token "
                                    "dynamic vs per-tensor static",
                        "per_m": dec["cs_cg"]}
    if llm:
        out["llm_int8"] = {"us": round(llm["ms"] * 1e3, 1), "int8_TOPS": round(llm["int8_tops"], 1),
                           "frac": round(llm["int8_tops"] / PEAK_INT8_TOPS, 4),
                           "n_outlier": llm["n_outlier"], "side_GFLOP": round(llm["side_flops"] / 1e9, 3)}
    if blk:
        out["decoder_block"] = {
            "workload": "QKV 4096->12288, O 4096->4096, gate+up 4096->28672, down 14336->4096; bf16 in/out",
            "prefill_us": round(blk["ms_prefill"] * 1e3, 1), "prefill_tokens": blk["tokens"],
            "prefill_TOPS": round(blk["prefill_ops"] / (blk["ms_prefill"] * 1e-3) / 1e12, 1),
            "prefill_frac": round(blk["prefill_ops"] / (blk["ms_prefill"] * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
            "decode_us_per_step": round(blk["ms_step"] * 1e3, 2), "decode_batch": blk["batch"],
            "decode_steps_per_replay": blk["steps"],
            "decode_GBps": round(blk["step_bytes"] / (blk["ms_step"] * 1e-3) / 1e9, 1),
            "decode_frac": round(blk["step_bytes"] / (blk["ms_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "int8_weight_MB": round(blk["weight_bytes"] / 1e6, 1)}
    if smq:
        out["silu_mul_quant"] = {
            "workload": f"h = SiLU(gate) * up, {smq['M']} tokens x {smq['K']} (gate and up: halves of one "
                        f"bf16 [M, 2K] buffer), per-token INT8; then the down projection {smq['K']}->{smq['N']}",
            "fused_us": round(smq["ms_fused"] * 1e3, 2),
            "fused_GBps": round(smq["bytes"] / (smq["ms_fused"] * 1e-3) / 1e9, 1),
            "fused_frac": round(smq["bytes"] / (smq["ms_fused"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_MB": round(smq["bytes"] / 1e6, 1),
            "unfused_torch_silu_mul_plus_quantizer_us": round(smq["ms_unfused"] * 1e3, 2),
            "down_projection_us": round(smq["ms_linear"] * 1e3, 1),
            "down_projection_TOPS": round(smq["ops"] / (smq["ms_linear"] * 1e-3) / 1e12, 1)}
    if not args.no_cpu_baseline:
        log("[cpu] timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(pre, synth, llm_host=llm.get("host") if llm else None, dec=dec)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
