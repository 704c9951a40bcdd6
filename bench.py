#!/usr/bin/env python3
"""Benchmark of the rotated low-bit linear layer on one MI355X.

Headline workload: the online W8A8 rotated linear at DiT image shape -- 4608 tokens (4096 latent
patches + 512 text tokens) x d_in 4096 -> d_out 16384 (the MLP-up linear of a 7B, 32-layer
single-stream DiT), bf16 activations in, bf16 out, INT8 weights rotated and quantised offline with
the same RPBH descriptor, both operands' codes in the product's tiled layout (RTQ_INT8_TILED; the
row-major format is timed beside it).  One step = one call of rtq_rotated_qlinear, one pass of the online path
over one batch:
    rotate-quantise (gather + sign + FWHT-64 + per-token INT8)   [HBM-bound]
    product         (INT8 MFMA product + scale epilogue)          [MFMA-bound]
The timed steps are bracketed by synchronisation only; each kernel's duration comes from the same
two launches issued separately (rtq_quantize_rows, rtq_qgemm) with HIP events around each on the
launching stream.

value      = 2*T*d_in*d_out per step / step time, in TFLOP/s (integer ops, i.e. TOP/s).
roofline   = the INT8 GEMM against the dense INT8 MFMA peak (5.0 POP/s); the RPBH+quantise kernel
             is reported against HBM (8 TB/s) in rpbh_roofline.
cpu_baseline = the CPU oracle (dense Pi product, int64 triple loop) on a bounded token sample,
             scaled linearly to the full step.
Also reported (extra): the offline weight rotate-quantise of one DiT block's four linears; the
W4A4, W3A3, W4A6 (4608x4096->4096) and W2A4 (4608x16384->4096) codebook layers; the W8A8 layer with
zero points; the transform ablation (block Hadamard without the permutation, dense Haar rotation).
Inputs are synthetic (seeded; see workloads/), resident in HBM before timing; the activations
rotate over enough copies (> 512 MB) that the 256 MB Infinity Cache cannot serve them.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "rotated W8A8 qlinear TFLOP/s (% INT8 MFMA peak) + RPBH-quantize GB/s (% HBM)"
PEAK_INT8_TOPS = 5000.0     # dense INT8 MFMA, MI355X
PEAK_F16_TFLOPS = 2500.0    # dense fp16/bf16 MFMA, MI355X
PEAK_HBM_GBPS = 8000.0      # HBM3E


def _bf16_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _copies(t, min_bytes, torch):
    n = max(3, -(-min_bytes // (t.numel() * t.element_size())))
    return [t.clone() for _ in range(n)]


def _prewarm(launch, torch, seconds=0.5):
    """Untimed: run `launch` until `seconds` of wall time have passed, so the GPU is at its steady
    clock and power state before the warm-up and timed steps (a cold GPU runs the first few hundred
    milliseconds of MFMA work measurably slower)."""
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            launch(i)
            i += 1
        torch.cuda.synchronize()
    return i


def _source_sha256(*names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "rotation_then_quantize_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# each kernel's source and the headers it includes: counters taken before any of them changed are stale
KERNEL_SOURCES = {"gemm_i8_kernel": ("gemm_i8.hip", "codebook_int8.h", "rtq_internal.h"),
                  "rpbh_wave_bf16_kernel": ("rpbh_quant.hip", "codebook_int8.h", "rtq_internal.h")}


def _traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs (scaled by the
    plain-copy calibration recorded with them), or None when the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != _source_sha256(*KERNEL_SOURCES[kernel]):
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def _time_pairs(steps, launch_a, launch_b, torch):
    """Run `steps` iterations of (a, b) with events around each launch on the current stream."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        launch_a(i)
        ev[i][1].record()
        launch_b(i)
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ta = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)])  # ms
    tb = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(steps)])
    return wall, ta, tb


def _burst_ms(n, launch, torch):
    """Per-launch duration of `n` back-to-back launches between two events on the current stream."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def bench_w8a8(args, torch, rtq, workloads, mode=None):
    """The headline step.  mode RTQ_INT8_TILED (default): weight and activation codes in the
    product's tiled layout; RTQ_INT8: row-major codes (reported beside it)."""
    mode = rtq.RTQ_INT8_TILED if mode is None else mode
    d, N = workloads.DIT_HIDDEN, workloads.DIT_MLP
    xh = workloads.dit_activations_bf16(d)
    T = xh.shape[0]
    wh = workloads.dit_weight_bf16("mlp_up")
    R = rtq.Rpbh.from_seed(workloads.RPBH_SEED[d], d)
    tiled = mode == rtq.RTQ_INT8_TILED
    w = _bf16_dev(wh, torch)
    wq = torch.empty(((rtq.tiled_rows(N) if tiled else N), d), dtype=torch.int8, device="cuda")
    ws = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(w, wq, ws, R, mode)                   # offline, not timed here
    del w
    xs = _copies(_bf16_dev(xh, torch), 512 << 20, torch)
    codes = torch.empty(((rtq.tiled_rows(T) if tiled else T), d), dtype=torch.int8, device="cuda")
    scale = torch.empty(T, dtype=torch.float32, device="cuda")
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")

    def quant(i):
        rtq.quantize_rows(xs[i % len(xs)], codes, scale, R, mode)

    split_ws = rtq.new_qgemm_workspace()

    def gemm(i):
        rtq.qgemm(codes, scale, wq, ws, y, d, mode, workspace=split_ws, n_tokens=T, n_out=N)

    # The timed steps: the layer's entry point (rotate-quantise, then the product, on one stream),
    # K launches bracketed by synchronisation only.
    ws_bytes = rtq.rotated_qlinear_workspace(T, d, mode)
    work = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

    def step(i):
        rtq.rotated_qlinear(xs[i % len(xs)], R, wq, ws, y, mode, workspace=work)

    prewarm = _prewarm(step, torch)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Per-kernel durations, from the same two launches issued separately with HIP events around
    # each on the launching stream (the event packets add a few us to each step's span, which is
    # why the steps above are timed without them).
    _, tq, tg = _time_pairs(args.steps, quant, gemm, torch)
    # The quantiser is short enough that the event packets around each launch add a few us to its
    # span; its per-launch duration is also taken over a burst of back-to-back launches (inputs
    # still rotating over the copies), which is what a kernel trace reports.
    quant_burst_ms = _burst_ms(max(20, args.steps), quant, torch)
    fused_ms = (float(tq.mean()) + float(tg.mean()))
    flops = 2.0 * T * d * N
    q_bytes = T * (2 * d + d + 4)                           # bf16 in, int8 codes out, fp32 scale out
    return {
        "T": T, "d": d, "N": N, "wall_s": wall, "step_ms": wall * 1e3 / args.steps,
        "quant_ms": float(tq.mean()), "gemm_ms": float(tg.mean()),
        "quant_ms_median": float(np.median(tq)), "gemm_ms_median": float(np.median(tg)),
        "quant_burst_ms": quant_burst_ms,
        "flops": flops, "quant_bytes": q_bytes, "kernel_sum_ms": fused_ms, "prewarm_steps": prewarm,
    }


def bench_offline(args, torch, rtq, workloads):
    """Offline rotate + INT8 quantise of one DiT block's four linears (bf16 in; int8 codes in the
    product's tiled layout + bf16 row scales out): the four launches back to back, and each linear
    alone (a burst of its launch), for the per-kernel roofline."""
    mats = []
    total = 0
    for name, n_out, d_in in workloads.DIT_LINEARS:
        w = _bf16_dev(workloads.dit_weight_bf16(name), torch)
        R = rtq.Rpbh.from_seed(workloads.RPBH_SEED[d_in], d_in)
        q = torch.empty((rtq.tiled_rows(n_out), d_in), dtype=torch.int8, device="cuda")
        s = torch.empty(n_out, dtype=torch.bfloat16, device="cuda")
        mats.append((name, w, R, q, s, n_out * d_in * 3 + n_out * 2))
        total += n_out * d_in * 3 + n_out * 2

    def launch(m):
        _, w, R, q, s, _ = m
        rtq.quantize_rows(w, q, s, R, rtq.RTQ_INT8_TILED)

    def run():
        for m in mats:
            launch(m)

    for _ in range(max(1, args.warmup // 2)):
        run()
    reps = max(3, args.steps // 5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    per = {}
    for m in mats:
        t = _burst_ms(max(5, reps), lambda i, m=m: launch(m), torch)
        per[m[0]] = {"ms": t, "bytes": m[5], "GB/s": m[5] / (t * 1e-3) / 1e9,
                     "frac_hbm": m[5] / (t * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    return {"bytes": total, "ms": ms, "GB/s": total / (ms * 1e-3) / 1e9,
            "frac_hbm": total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, "per_linear": per,
            "codes_layout": "tiled (RTQ_INT8_TILED)"}


def bench_codebook(args, torch, rtq, workloads, variant, mode=None):
    """One online codebook layer (quantise + product).  mode RTQ_CODEBOOK_I8_TILED (default): codes
    on the INT8 matrix cores (int8 codebook values, 1 byte per activation element), both operands
    in the tiled layouts; RTQ_CODEBOOK_I8: the same with row-major operands; RTQ_CODEBOOK: fp16 LUT
    product."""
    mode = rtq.RTQ_CODEBOOK_I8_TILED if mode is None else mode
    tiled = mode == rtq.RTQ_CODEBOOK_I8_TILED
    i8 = mode in (rtq.RTQ_CODEBOOK_I8, rtq.RTQ_CODEBOOK_I8_TILED)
    bits_a = 4
    if variant in ("w4a4", "w3a3", "w4a6"):     # the attention-output shape
        d, N = workloads.DIT_HIDDEN, workloads.DIT_HIDDEN
        bits_w, bits_a = {"w4a4": (4, 4), "w3a3": (3, 3), "w4a6": (4, 6)}[variant]
        wh = workloads.w4a4_weight_bf16()
    else:
        d, N, bits_w = workloads.DIT_MLP, workloads.DIT_HIDDEN, 2
        wh = workloads.w2a4_weight_bf16()
    xh = workloads.dit_activations_bf16(d)
    T = xh.shape[0]
    R = rtq.Rpbh.from_seed(workloads.RPBH_SEED[d], d)
    cb_a, cb_w = rtq.Codebook.for_dim(d, bits_a), rtq.Codebook.for_dim(d, bits_w)
    w = _bf16_dev(wh, torch)
    wmode = rtq.RTQ_CODEBOOK_TILED if tiled else rtq.RTQ_CODEBOOK
    wc = torch.empty(rtq.tiled_code_bytes(N, d, wmode, bits_w) or N * d * bits_w // 8, dtype=torch.uint8, device="cuda")
    wn = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(w, wc, wn, R, wmode, cb_w, 0.0)
    del w
    xs = _copies(_bf16_dev(xh, torch), 512 << 20, torch)
    codes = torch.empty(rtq.tiled_rows(T) * d if tiled else T * (d if i8 else d * bits_a // 8),
                        dtype=torch.int8 if i8 else torch.uint8, device="cuda")
    norm = torch.empty(T, dtype=torch.float32, device="cuda")
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")

    def quant(i):
        rtq.quantize_rows(xs[i % len(xs)], codes, norm, R, mode, cb_a, 1e-8)

    split_ws = rtq.new_qgemm_workspace()

    def gemm(i):
        rtq.qgemm(codes, norm, wc, wn, y, d, mode, cb_a, cb_w, workspace=split_ws, n_tokens=T, n_out=N)

    _prewarm(lambda i: (quant(i), gemm(i)), torch, 0.25)
    for i in range(args.warmup):
        quant(i)
        gemm(i)
    steps = max(5, args.steps // 2)
    wall, tq, tg = _time_pairs(steps, quant, gemm, torch)
    quant_burst = _burst_ms(max(20, steps), quant, torch)
    flops = 2.0 * T * d * N
    q_bytes = T * (2 * d + (d if i8 else d * bits_a // 8) + 4)
    q_bytes_packed = T * (2 * d + d * bits_a // 8 + 4)   # the method's bytes: codes packed to bits_a
    gemm_tflops = flops / (tg.mean() * 1e-3) / 1e12
    peak = PEAK_INT8_TOPS if i8 else PEAK_F16_TFLOPS
    name = ("codebook on INT8 MFMA (int8 codebook values)" + (", tiled operands" if tiled else ", row-major operands")
            if i8 else "codebook, fp16 LUT on fp16 MFMA")
    return {"mode": name,
            "T": T, "d": d, "N": N, "bits_w": bits_w, "bits_a": bits_a, "step_ms": wall * 1e3 / steps,
            "quant_ms": quant_burst,
            "quant_event_span_ms": float(tq.mean()),
            "gemm_ms": float(tg.mean()), "TFLOP/s": flops / (wall / steps) / 1e12,
            "gemm_TFLOP/s": gemm_tflops, "gemm_peak": peak, "gemm_frac_peak": gemm_tflops / peak,
            "rpbh_bytes": q_bytes, "rpbh_GB/s": q_bytes / (quant_burst * 1e-3) / 1e9,
            "rpbh_frac_hbm": q_bytes / (quant_burst * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "rpbh_bytes_packed_codes": q_bytes_packed,
            "rpbh_frac_hbm_packed_codes": q_bytes_packed / (quant_burst * 1e-3) / 1e9 / PEAK_HBM_GBPS}


def bench_w8a8_asym(args, torch, rtq, workloads):
    """The W8A8 DiT layer with asymmetric INT8 (a scale and a zero point per row) on both operands:
    the zero-point quantiser (bf16 weight scales offline, fp32 token scales online) and the product
    with its zero-point correction in the epilogue."""
    d, N = workloads.DIT_HIDDEN, workloads.DIT_MLP
    xh = workloads.dit_activations_bf16(d)
    T = xh.shape[0]
    R = rtq.Rpbh.from_seed(workloads.RPBH_SEED[d], d)
    w = _bf16_dev(workloads.dit_weight_bf16("mlp_up"), torch)
    wq = torch.empty((N, d), dtype=torch.int8, device="cuda")
    ws_ = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    wz = torch.empty(N, dtype=torch.int32, device="cuda")
    wsum = torch.empty(N, dtype=torch.int32, device="cuda")
    rtq.quantize_rows_asym(w, wq, ws_, wz, wsum, R)
    del w
    xs = _copies(_bf16_dev(xh, torch), 512 << 20, torch)
    codes = torch.empty((T, d), dtype=torch.int8, device="cuda")
    scale = torch.empty(T, dtype=torch.float32, device="cuda")
    zero = torch.empty(T, dtype=torch.int32, device="cuda")
    csum = torch.empty(T, dtype=torch.int32, device="cuda")
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    split_ws = rtq.new_qgemm_workspace()

    def quant(i):
        rtq.quantize_rows_asym(xs[i % len(xs)], codes, scale, zero, csum, R)

    def gemm(i):
        rtq.qgemm_asym(codes, scale, zero, csum, wq, ws_, wz, wsum, y, d, workspace=split_ws)

    _prewarm(lambda i: (quant(i), gemm(i)), torch, 0.25)
    for i in range(args.warmup):
        quant(i)
        gemm(i)
    steps = max(5, args.steps // 2)
    wall, tq, tg = _time_pairs(steps, quant, gemm, torch)
    quant_burst = _burst_ms(max(20, steps), quant, torch)
    flops = 2.0 * T * d * N
    q_bytes = T * (2 * d + d + 12)
    return {"T": T, "d": d, "N": N, "step_ms": wall * 1e3 / steps, "quant_ms": quant_burst,
            "quant_event_span_ms": float(tq.mean()), "gemm_ms": float(tg.mean()),
            "TFLOP/s": flops / (wall / steps) / 1e12, "gemm_TFLOP/s": flops / (tg.mean() * 1e-3) / 1e12,
            "gemm_frac_peak": flops / (tg.mean() * 1e-3) / 1e12 / PEAK_INT8_TOPS,
            "rpbh_bytes": q_bytes, "rpbh_GB/s": q_bytes / (quant_burst * 1e-3) / 1e9}


def bench_ablation(args, torch, rtq, workloads):
    """The transform ablation at the W8A8 DiT shape (OrbitQuant article, sections 2.3 and 3.3): RPBH
    against block Hadamard without the permutation (perm = identity, same signs) and against a dense
    Haar rotation applied as a bf16 GEMM (the vendor library, hipBLASLt through torch.matmul).
    Times: rotate-and-quantise launches and rotation alone, each a burst over rotating input
    copies. Quality: relative Frobenius error of the W8A8 output against the exact fp64 product on
    64 sampled tokens, with the workload's outlier channels spread as drawn and packed into the first
    blocks (the same column order applied to x and W leaves W x unchanged)."""
    d, N = workloads.DIT_HIDDEN, workloads.DIT_MLP
    xh = workloads.dit_activations_bf16(d)
    T = xh.shape[0]
    seed = workloads.RPBH_SEED[d]
    R = rtq.Rpbh.from_seed(seed, d)
    BH = rtq.Rpbh.without_permutation(seed, d)
    Q = torch.from_numpy(workloads.haar_orthogonal(seed, d)).cuda()
    Qt16 = Q.t().contiguous().to(torch.bfloat16)
    xs = _copies(_bf16_dev(xh, torch), 512 << 20, torch)
    codes = torch.empty((T, d), dtype=torch.int8, device="cuda")
    scale = torch.empty(T, dtype=torch.float32, device="cuda")
    rot16 = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    n = max(20, args.steps)

    def quant(desc):
        return lambda i: rtq.quantize_rows(xs[i % len(xs)], codes, scale, desc, rtq.RTQ_INT8)

    def dense_rotate(i):
        torch.matmul(xs[i % len(xs)], Qt16, out=rot16)

    def dense_rotate_quant(i):
        dense_rotate(i)
        rtq.quantize_rows(rot16, codes, scale, None, rtq.RTQ_INT8)

    def rpbh_rotate(i):
        rtq.rpbh_rotate(xs[i % len(xs)], rot16, R)

    for f in (quant(R), quant(BH), dense_rotate_quant, rpbh_rotate):
        _prewarm(f, torch, 0.1)
    t = {"rpbh_quantize_ms": _burst_ms(n, quant(R), torch),
         "block_hadamard_quantize_ms": _burst_ms(n, quant(BH), torch),
         "dense_rotate_then_quantize_ms": _burst_ms(n, dense_rotate_quant, torch),
         "rpbh_rotate_only_ms": _burst_ms(n, rpbh_rotate, torch),
         "dense_rotate_only_ms": _burst_ms(n, dense_rotate, torch)}
    t["dense_over_rpbh_rotate_only"] = t["dense_rotate_only_ms"] / t["rpbh_rotate_only_ms"]
    t["dense_over_rpbh_rotate_quantize"] = t["dense_rotate_then_quantize_ms"] / t["rpbh_quantize_ms"]
    t["block_hadamard_over_rpbh"] = t["block_hadamard_quantize_ms"] / t["rpbh_quantize_ms"]
    del xs

    # quality on 64 sampled tokens
    rows = np.sort(np.random.default_rng(9).choice(T, 64, replace=False))
    x32 = workloads.bf16_bits_to_f32(xh[rows])
    w32 = workloads.bf16_bits_to_f32(workloads.dit_weight_bf16("mlp_up"))
    quality = {}
    for layout in ("spread", "clustered"):
        order = (np.arange(d) if layout == "spread"
                 else workloads.clustered_order(d, workloads.dit_activation_outlier_channels(d)))
        xo = np.ascontiguousarray(x32[:, order])
        wo = np.ascontiguousarray(w32[:, order])
        ref = xo.astype(np.float64) @ wo.astype(np.float64).T
        xd, wd = torch.from_numpy(xo).cuda(), torch.from_numpy(wo).cuda()
        errs = {}
        for name in ("none", "block_hadamard", "rpbh", "dense_haar"):
            desc = {"none": None, "block_hadamard": BH, "rpbh": R, "dense_haar": None}[name]
            xin, win = xd, wd
            if name == "dense_haar":
                xin, win = xd @ Q.t(), wd @ Q.t()     # rotated in fp32
            wq = torch.empty((N, d), dtype=torch.int8, device="cuda")
            wsc = torch.empty(N, dtype=torch.float32, device="cuda")
            rtq.quantize_rows(win, wq, wsc, desc, rtq.RTQ_INT8)
            aq = torch.empty((len(rows), d), dtype=torch.int8, device="cuda")
            asc = torch.empty(len(rows), dtype=torch.float32, device="cuda")
            rtq.quantize_rows(xin, aq, asc, desc, rtq.RTQ_INT8)
            y = torch.empty((len(rows), N), dtype=torch.float32, device="cuda")
            rtq.qgemm(aq, asc, wq, wsc, y, d)
            torch.cuda.synchronize()
            errs[name] = float(np.linalg.norm(y.cpu().numpy() - ref) / np.linalg.norm(ref))
        quality[layout] = errs
    return {"shape": f"{T}x{d} activations (rotation), {T}x{d}->{N} (quality, 64 tokens)", **t,
            "w8a8_rel_error": quality}


def cpu_baseline(workloads):
    """The oracle, as written, on a bounded token sample of the W8A8 step, scaled to the full step:
    per-token online cost (dense Pi rotation + INT8 quantise) and per-(token, channel) GEMM cost are
    measured on the sample and extrapolated linearly to 4608 tokens x 16384 channels."""
    import oracle
    d, N = workloads.DIT_HIDDEN, workloads.DIT_MLP
    xh = workloads.dit_activations_bf16(d)
    T = xh.shape[0]
    perm, signs = oracle.rpbh_descriptor(workloads.RPBH_SEED[d], d)
    pi = oracle.rpbh_dense(d, 64, perm, signs)              # set-up, once per d: not timed
    tok = T                                                 # the whole step: no extrapolation
    ch = N
    wsamp = workloads.bf16_bits_to_f32(workloads.dit_weight_bf16("mlp_up")[:ch])
    wq = oracle.weights_int8(wsamp, pi, True)               # offline: not timed
    x = workloads.bf16_bits_to_f32(xh[:tok])
    t0 = time.perf_counter()
    act = oracle.activations_int8(x, pi)
    t1 = time.perf_counter()
    acc = oracle.gemm_int8(act["q"], wq["q"])
    oracle.rescale_int8(acc, act["scale"], wq["scale"])
    t2 = time.perf_counter()
    per_token = (t1 - t0) / tok
    per_dot = (t2 - t1) / (tok * ch)
    full = T * per_token + T * N * per_dot
    return {"value": 2.0 * T * d * N / full / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{tok} of the {T} tokens through the oracle's online W8A8 path (dense Pi product, INT8 "
                      f"quantise, int64 triple-loop GEMM against {ch} weight rows, rescale); weights rotated and "
                      f"quantised by the oracle beforehand (untimed); {full:.1f} s for the step",
            "sample_seconds": t2 - t0}


COPY_BYTES = 256 << 20


def _counter_per_dispatch(run_dir, counter):
    """{kernel name: [value per dispatch]} for one counter from a rocprofv3 CSV output directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                key = (row["Kernel_Name"], row["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (name, _), v in sorted(per.items(), key=lambda kv: int(kv[0][1])):
        out.setdefault(name, []).append(v)
    return out


def write_traffic(fetch_dir, write_dir):
    """HBM bytes per launch of the hot kernels = FETCH_SIZE / WRITE_SIZE (KiB per dispatch, median over
    dispatches) x the factor that maps the same counter to the known bytes of the plain copy."""
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")

    def pick(table, key):
        vals = [v for name, vs in table.items() if key in name for v in vs]
        if not vals:
            raise SystemExit(f"no dispatch of a kernel named *{key}* in the counter data")
        return float(np.median(vals)) * 1024.0

    f_copy, w_copy = pick(fetch, "bitwise_not"), pick(write, "bitwise_not")
    cal = {"kernel": "bitwise_not over int8 (elementwise)", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
           "fetch_counter_bytes": f_copy, "write_counter_bytes": w_copy,
           "fetch_factor": COPY_BYTES / f_copy, "write_factor": COPY_BYTES / w_copy}
    kernels = {}
    for kernel in KERNEL_SOURCES:
        fb, wb = pick(fetch, kernel), pick(write, kernel)
        kernels[kernel] = {"source_sha256": _source_sha256(*KERNEL_SOURCES[kernel]),
                           "fetch_counter_bytes": fb, "write_counter_bytes": wb,
                           "fetch_bytes": round(fb * cal["fetch_factor"]), "write_bytes": round(wb * cal["write_factor"])}
    rec = {"note": "HBM bytes per launch of the W8A8 step's kernels (4608 x 4096 -> 16384, bf16 in/out), from "
                   "rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs of 'bench.py --calibrate-copy --only w8a8', "
                   "each scaled by the factor that maps the same counter to the known bytes of a plain copy",
           "calibration": cal, "kernels": kernels}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--only", choices=["w8a8", "codebook", "ablation", "asym", "offline", "all"], default="all",
                    help="w8a8: time only the headline step (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain streaming kernel of known size (bitwise_not over 256 MiB of int8, "
                         "5 times) so a rocprofv3 FETCH_SIZE/WRITE_SIZE run can be scaled to bytes")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: read the counter CSVs of a FETCH_SIZE run and a WRITE_SIZE run of "
                         "'bench.py --calibrate-copy --only w8a8' and write profiles/traffic.json")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the rotated linear is measured at "
                                   "its single-GPU shape; multi-GPU sharding is not implemented",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import rotation_then_quantize_amd as rtq
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    rtq.load_library()

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES, dtype=torch.int8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if args.only == "asym":
        print(json.dumps(bench_w8a8_asym(args, torch, rtq, workloads)))
        return
    if args.only == "offline":   # the offline weight rotate-quantise only (profiling runs)
        print(json.dumps(bench_offline(args, torch, rtq, workloads)))
        return
    if args.only == "ablation":
        print(json.dumps(bench_ablation(args, torch, rtq, workloads)))
        return
    if args.only == "codebook":   # the codebook layers only (profiling runs)
        out = {k: bench_codebook(args, torch, rtq, workloads, v) for k, v in
               [("w4a4_dit_attn_out_4608x4096x4096", "w4a4"), ("w2a4_dit_mlp_down_4608x16384x4096", "w2a4"),
                ("w3a3_dit_attn_out_4608x4096x4096", "w3a3"), ("w4a6_dit_attn_out_4608x4096x4096", "w4a6")]}
        print(json.dumps(out))
        return
    r = bench_w8a8(args, torch, rtq, workloads)
    extra = {}
    if args.only == "all":
        rm = bench_w8a8(args, torch, rtq, workloads, rtq.RTQ_INT8)
        extra["w8a8_row_major_codes"] = {k: rm[k] for k in ("step_ms", "quant_ms", "gemm_ms", "quant_burst_ms")}
        extra["offline_weight_rotate_quantize"] = bench_offline(args, torch, rtq, workloads)
        extra["w4a4_dit_attn_out_4608x4096x4096"] = bench_codebook(args, torch, rtq, workloads, "w4a4")
        extra["w2a4_dit_mlp_down_4608x16384x4096"] = bench_codebook(args, torch, rtq, workloads, "w2a4")
        for k, v in (("w4a4_dit_attn_out_4608x4096x4096", "w4a4"), ("w2a4_dit_mlp_down_4608x16384x4096", "w2a4")):
            rm = bench_codebook(args, torch, rtq, workloads, v, rtq.RTQ_CODEBOOK_I8)
            extra[k + "_row_major"] = {f: rm[f] for f in ("step_ms", "quant_ms", "gemm_ms", "gemm_frac_peak")}
        extra["w4a4_dit_attn_out_4608x4096x4096_fp16_lut"] = bench_codebook(args, torch, rtq, workloads, "w4a4",
                                                                            rtq.RTQ_CODEBOOK)
        extra["w2a4_dit_mlp_down_4608x16384x4096_fp16_lut"] = bench_codebook(args, torch, rtq, workloads, "w2a4",
                                                                             rtq.RTQ_CODEBOOK)
        extra["w3a3_dit_attn_out_4608x4096x4096"] = bench_codebook(args, torch, rtq, workloads, "w3a3")
        extra["w4a6_dit_attn_out_4608x4096x4096"] = bench_codebook(args, torch, rtq, workloads, "w4a6")
        extra["w8a8_asym_dit_mlp_up_4608x4096x16384"] = bench_w8a8_asym(args, torch, rtq, workloads)
        extra["transform_ablation"] = bench_ablation(args, torch, rtq, workloads)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(workloads)

    step_s = r["step_ms"] * 1e-3
    value = r["flops"] / step_s / 1e12
    gemm_tops = r["flops"] / (r["gemm_ms"] * 1e-3) / 1e12
    q_gbps = r["quant_bytes"] / (r["quant_burst_ms"] * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "w8a8_dit_mlp_up_4608x4096x16384_bf16", "tokens": r["T"], "d_in": r["d"],
                   "d_out": r["N"], "io": "bf16", "weights": "int8 per-row, bf16 scales",
                   "codes_layout": "tiled (RTQ_INT8_TILED: 256-row x 64-byte blocks)",
                   "activations": "int8 per-token, fp32 scales", "rotation": "RPBH h=64"},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tops / PEAK_INT8_TOPS, 4), "traffic": _traffic("gemm_i8_kernel"),
                     "kernel": "gemm_i8_kernel", "work_per_launch": r["flops"], "avg_ms": round(r["gemm_ms"], 5),
                     "median_ms": round(r["gemm_ms_median"], 5)},
        "rpbh_roofline": {"bound": "hbm", "achieved": round(q_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                          "frac": round(q_gbps / PEAK_HBM_GBPS, 4), "traffic": _traffic("rpbh_wave_bf16_kernel"),
                          "kernel": "rpbh_wave_bf16_kernel (int8)", "bytes_per_launch": r["quant_bytes"],
                          "avg_ms": round(r["quant_burst_ms"], 5),
                          "event_span_avg_ms": round(r["quant_ms"], 5),
                          "event_span_median_ms": round(r["quant_ms_median"], 5)},
        "kernel_event_spans_ms_per_step": round(r["kernel_sum_ms"], 4),
        "cpu_baseline": None if cpu is None else {k: (round(v, 6) if isinstance(v, float) else v)
                                                 for k, v in cpu.items()},
    }
    if extra:
        out["extra"] = extra
    print(json.dumps(out))


if __name__ == "__main__":
    main()
