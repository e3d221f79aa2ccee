#!/usr/bin/env python3
"""Benchmark of the quantized INT8 linear layer on one MI355X.

One step = one forward of the W8A8 layer on the largest single-GPU workload,
the 530B-class FFN-up column slice (one GPU's share of a tensor-parallel
layer): fused smoothing (alpha 0.7) + per-token quantization of X
[4096 x 20480] fp16, then the int8 MFMA GEMM against the per-tensor-quantized
W [10240 x 20480] with the dequant epilogue writing fp16 Y.  Weight
preparation (calibration, smoothing factors, weight quantization) happens once,
before the timed region.  Inputs are resident in HBM when timing starts.

Before the W warm-up steps the step runs untimed for at least 0.5 s of GPU time
(the shader clock settles over that time); the JSON line reports how many
steps that took (clock_settle_steps) and the p10/p50/p90 of single-step times
beside the mean over the K timed steps, which is `value`.

value = 2*M*N*K / step time, in TOPS, quantization included; the timed steps
have no events between their kernels.
roofline: the GEMM kernel (for this shape two launches of the same kernel:
256 x 256 tiles over the first 8192 output columns, 128 x 128 tiles over the
last 2048), algorithmic 2MNK ops per call over the call's average duration
(HIP events around each call, recorded on the stream the library launches on,
over a second timed pass of the same steps), against the 5.0 POP/s dense int8
MFMA peak.
cpu_baseline: the CPU oracle doing the same per-token work on a bounded number
of token rows, on this host's cores.
secondary: the 7B prefill projections, decode (GB/s), LLM.int8(), zero-point
activations, LayerNorm + quantization, static scale, FP8 and KV-cache workloads,
same method.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W8A8 linear TOPS incl. quant+dequant (% int8 MFMA peak); decode GB/s (% HBM peak)"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_FP8_TOPS = 5000.0       # MI355X dense fp8 MFMA, 5.0 PFLOP/s
PEAK_FP16_TFLOPS = 2500.0    # MI355X dense fp16 MFMA, 2.5 PFLOP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
GEMM_SRC = os.path.join(ROOT, "int8_quantization_amd", "csrc", "gemm.hip")
GEMV_SRC = os.path.join(ROOT, "int8_quantization_amd", "csrc", "gemv.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_for(key, src):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, if the kernel source is unchanged since the counters were taken."""
    try:
        t = json.load(open(TRAFFIC_FILE)).get(key)
    except (OSError, ValueError):
        return None
    if not t or t.get("source_sha") != sha(src):
        return None
    return t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]


class Timer:
    """Events recorded on torch's current stream, which is the stream every
    library call launches on."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def around(self, fn):
        a = self.torch.cuda.Event(enable_timing=True)
        b = self.torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.append((a, b))

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(1, len(self.pairs))


def time_steps(torch, step, steps, warmup, kernel_events=True):
    """ms per step over `steps` steps after `warmup`, and the mean duration of
    the launches the step brackets with its timer (None when kernel_events is
    False: then no per-kernel events sit in the timed region)."""
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    timer = Timer(torch) if kernel_events else None
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        step(timer)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, (timer.mean_ms() if timer else None)


def step_percentiles(torch, step, n):
    """p10 / p50 / p90 of single-step times (ms): HIP events between steps only."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record()
    for i in range(n):
        step(None)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
    return dict(p10=float(np.percentile(t, 10)), p50=float(np.percentile(t, 50)), p90=float(np.percentile(t, 90)))


def shader_clock():
    """The current shader clock level from the amdgpu driver's sysfs table (a plain
    file read; the line marked '*' is the active level).  Best effort."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return line.split(":", 1)[1].strip(" *\n")
        except OSError:
            continue
    return "unavailable"


def gpu_info(torch):
    """Device name, CU count and the shader clock level read right after the timed
    steps (a snapshot, not the sustained clock)."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "cus": p.multi_processor_count, "sclk_after_timing": shader_clock()}


def settle(torch, step, seconds=0.5, min_steps=20, max_steps=5000):
    """Run the step untimed until `seconds` of GPU time have passed (the shader clock
    ramps up over roughly that long); returns the number of steps run."""
    n, batch = 0, min_steps
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    while n < max_steps:
        for _ in range(batch):
            step(None)
        n += batch
        t1.record()
        torch.cuda.synchronize()
        if t0.elapsed_time(t1) >= seconds * 1e3:
            break
    return n


def prepare_weight(torch, sq, d, X_cal, W, alpha, gran):
    """Offline: calibration max, smoothing factors, smoothed weight quantization (GPU)."""
    N, K = W.shape
    act = torch.zeros(K, dtype=torch.float32, device="cuda")
    s = torch.empty(K, dtype=torch.float32, device="cuda")
    W_d = d(W)
    if alpha is None:
        s = None
    else:
        sq.sq_smooth_scales(d(X_cal), W_d, alpha, act, s)
    Wq = torch.empty(N, K, dtype=torch.int8, device="cuda")
    ws = torch.empty(N if gran == 0 else 1, dtype=torch.float32, device="cuda")
    wsp = torch.empty(sq.sq_workspace_size(sq.SQ_OP_QUANT_WEIGHT, 0, N, K), dtype=torch.uint8, device="cuda")
    sq.sq_quantize_weight(W_d, s, gran, Wq, ws, wsp)
    torch.cuda.synchronize()
    del W_d
    return s, Wq, ws


def bench_w8a8(torch, sq, d, wl, steps, warmup, settle_s=0.5):
    """Prefill-style W8A8 forward over every weight of the workload."""
    M, K = wl.X.shape
    X = d(wl.X)
    projs = []
    for name, W in wl.weights.items():
        s, Wq, ws = prepare_weight(torch, sq, d, wl.calib, W, wl.alpha, wl.gran)
        Y = torch.empty(M, W.shape[0], dtype=torch.float16 if wl.out_dtype == np.float16 else torch.float32,
                        device="cuda")
        projs.append((name, s, Wq, ws, Y))
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")

    def step(timer):
        for _, s, Wq, ws, Y in projs:
            sq.sq_quantize_per_token(X, s, Xq, xs)
            g = lambda: sq.w8a8_gemm_dequant(Xq, xs, Wq, ws, wl.gran, None, Y)
            timer.around(g) if timer else g()

    settled = settle(torch, step, settle_s)
    # the step as a user runs it (no events between its kernels), then the same steps again
    # with HIP events around each GEMM call for the kernel's average duration
    ms, _ = time_steps(torch, step, steps, warmup, kernel_events=False)
    pct = step_percentiles(torch, step, steps)
    _, gemm_ms = time_steps(torch, step, steps, 5)
    # the fused smoothing + per-token quantizer on its own (2MK + MK + 4M bytes)
    s0 = projs[0][1]
    q_ms, _ = time_steps(torch, lambda t: sq.sq_quantize_per_token(X, s0, Xq, xs), steps, 5, kernel_events=False)
    qb = X.element_size() * M * K + M * K + 4 * M
    ops = sum(2.0 * M * p[2].shape[0] * K for p in projs)
    fp16 = fp16_reference(torch, d, wl, X, steps, warmup, ops, ms) if wl.X.dtype == np.float16 else None
    return dict(ms=ms, gemm_ms=gemm_ms, ops=ops, gemm_ops_per_launch=ops / len(projs),
                Ns=[p[2].shape[0] for p in projs], pct=pct, settle_steps=settled,
                quantize=dict(us=q_ms * 1e3, GBps=qb / (q_ms * 1e-3) / 1e9,
                              hbm_frac=qb / (q_ms * 1e-3) / 1e9 / PEAK_HBM_GBS),
                fp16_reference=fp16)


def fp16_reference(torch, d, wl, X, steps, warmup, ops, w8a8_ms):
    """The same projections as an unquantized fp16 layer, Y = X W^T through torch.mm
    (the vendor GEMM library), timed like the W8A8 step: the pages quote W8A8
    speed-ups over fp16 (1.5-2x), and this is that ratio on this GPU.  Context only: it
    is not part of the path and no output of it is checked."""
    Ws = [d(W) for W in wl.weights.values()]
    Ys = [torch.empty(X.shape[0], W.shape[0], dtype=torch.float16, device="cuda") for W in Ws]

    def step(_):
        for W, Y in zip(Ws, Ys):
            torch.mm(X, W.t(), out=Y)

    settle(torch, step, 0.3)
    ms, _ = time_steps(torch, step, steps, warmup, kernel_events=False)
    del Ws, Ys
    torch.cuda.empty_cache()
    tflops = ops / (ms * 1e-3) / 1e12
    return dict(ms_per_step=round(ms, 5), TFLOPs=round(tflops, 1), fp16_mfma_frac=round(tflops / PEAK_FP16_TFLOPS, 4),
                w8a8_speedup=round(ms / w8a8_ms, 3), call="torch.mm(X, W.t(), out=Y), fp16 in and out")


def bench_fp8(torch, sq, d, wl, steps, warmup):
    """The headline prefill step with FP8 E4M3 codes instead of int8: per-token FP8
    quantization and the FP8 GEMM + dequant epilogue for each projection (same shapes,
    smoothing and per-channel weight scales)."""
    M, K = wl.X.shape
    X = d(wl.X)
    projs = []
    for name, W in wl.weights.items():
        N = W.shape[0]
        act = torch.zeros(K, dtype=torch.float32, device="cuda")
        s = torch.empty(K, dtype=torch.float32, device="cuda")
        W_d = d(W)
        sq.sq_smooth_scales(d(wl.calib), W_d, wl.alpha, act, s)
        Wq = torch.empty(N, K, dtype=torch.uint8, device="cuda")
        ws = torch.empty(N, dtype=torch.float32, device="cuda")
        sq.sq_quantize_weight_fp8(W_d, s, 0, Wq, ws)
        del W_d
        projs.append((s, Wq, ws, torch.empty(M, N, dtype=torch.float16, device="cuda")))
    Xq = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")

    def step(timer):
        for s, Wq, ws, Y in projs:
            sq.sq_quantize_per_token_fp8(X, s, Xq, xs)
            g = lambda: sq.fp8_gemm_dequant(Xq, xs, Wq, ws, 0, None, Y)
            timer.around(g) if timer else g()

    ms, _ = time_steps(torch, step, steps, warmup, kernel_events=False)
    _, gemm_ms = time_steps(torch, step, steps, 5)
    ops = sum(2.0 * M * p[1].shape[0] * K for p in projs)
    gemm_tops = ops / len(projs) / (gemm_ms * 1e-3) / 1e12
    return dict(ms_per_step=ms, TOPS=ops / (ms * 1e-3) / 1e12, gemm_us_per_launch=gemm_ms * 1e3,
                gemm_TOPS=gemm_tops, gemm_mfma_frac=gemm_tops / PEAK_FP8_TOPS)


def bench_zero_point(torch, sq, d, wl, steps, warmup, sample_rows=64):
    """Zero-point activations on the 7B FFN-down projection over SiLU outputs: the step
    (zero-point per-token quantization + the GEMM with the row-sum correction) beside the
    symmetric step on the same input, and, on a sample of rows, the error of both against
    the unquantized fp64 product (as SNR in dB: zero points are for ranges not centred on 0)."""
    M, K = wl.X.shape
    W = wl.weights["down"]
    N = W.shape[0]
    X = d(wl.X)
    _, Wq, ws = prepare_weight(torch, sq, d, wl.calib, W, None, 0)
    rs = torch.empty(N, dtype=torch.int32, device="cuda")
    sq.sq_weight_rowsum(Wq, rs)
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")
    xz = torch.empty(M, dtype=torch.int32, device="cuda")
    Ya = torch.empty(M, N, dtype=torch.float16, device="cuda")
    Ys = torch.empty(M, N, dtype=torch.float16, device="cuda")

    def step_asym(timer):
        sq.sq_quantize_per_token_asym(X, None, Xq, xs, xz)
        sq.w8a8_asym_gemm_dequant(Xq, xs, xz, Wq, ws, 0, rs, None, Ya)

    def step_sym(timer):
        sq.sq_quantize_per_token(X, None, Xq, xs)
        sq.w8a8_gemm_dequant(Xq, xs, Wq, ws, 0, None, Ys)

    settle(torch, step_asym, 0.3)
    ms_a, _ = time_steps(torch, step_asym, steps, warmup, kernel_events=False)
    ms_s, _ = time_steps(torch, step_sym, steps, warmup, kernel_events=False)
    q_ms, _ = time_steps(torch, lambda t: sq.sq_quantize_per_token_asym(X, None, Xq, xs, xz), steps, 5,
                         kernel_events=False)
    step_asym(None)
    step_sym(None)
    torch.cuda.synchronize()
    ref = wl.X[:sample_rows].astype(np.float64) @ W.astype(np.float64).T

    def snr(Y):
        e = Y[:sample_rows].float().cpu().numpy().astype(np.float64) - ref
        return float(10 * np.log10((ref ** 2).sum() / (e ** 2).sum()))

    ops = 2.0 * M * N * K
    qb = 2 * M * K + M * K + 8 * M
    return dict(workload=wl.name, ms_per_step=ms_a, TOPS=ops / (ms_a * 1e-3) / 1e12,
                symmetric_ms_per_step=ms_s, symmetric_TOPS=ops / (ms_s * 1e-3) / 1e12,
                quantize_us=q_ms * 1e3, quantize_hbm_frac=qb / (q_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                snr_db_vs_fp64=snr(Ya), symmetric_snr_db_vs_fp64=snr(Ys), snr_rows=sample_rows)


def bench_fp8_decode(torch, sq, d, wl, steps, warmup, copies=3):
    """FP8 decode rows (M in {1,4,16}) of the 70B FFN-up weight: per-token FP8 codes
    and the FP8 weight-streaming kernel, three rotated weight copies."""
    W = wl.weights["w"]
    N, K = W.shape
    act = torch.zeros(K, dtype=torch.float32, device="cuda")
    s = torch.empty(K, dtype=torch.float32, device="cuda")
    W_d = d(W)
    sq.sq_smooth_scales(d(wl.calib), W_d, wl.alpha, act, s)
    Wq0 = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    ws = torch.empty(N, dtype=torch.float32, device="cuda")
    sq.sq_quantize_weight_fp8(W_d, s, 0, Wq0, ws)
    del W_d
    Wqs = [Wq0] + [Wq0.clone() for _ in range(copies - 1)]
    out = {}
    for M in wl.decode_rows:
        X = d(wl.X[:M])
        Xq = torch.empty(M, K, dtype=torch.uint8, device="cuda")
        xs = torch.empty(M, dtype=torch.float32, device="cuda")
        Y = torch.empty(M, N, dtype=torch.float16, device="cuda")
        it = [0]

        def step(timer):
            Wq = Wqs[it[0] % copies]
            it[0] += 1
            sq.sq_quantize_per_token_fp8(X, s, Xq, xs)
            g = lambda: sq.fp8_gemm_dequant(Xq, xs, Wq, ws, 0, None, Y)
            timer.around(g) if timer else g()

        ms, _ = time_steps(torch, step, steps, warmup, kernel_events=False)
        _, gemv_ms = time_steps(torch, step, steps, 2)

        def gemv_only(timer):
            Wq = Wqs[it[0] % copies]
            it[0] += 1
            sq.fp8_gemm_dequant(Xq, xs, Wq, ws, 0, None, Y)

        b2b_ms, _ = time_steps(torch, gemv_only, steps, 2, kernel_events=False)
        gemv_bytes = N * K + 4 * N + M * K + 4 * M + 2 * M * N
        out[f"M{M}"] = dict(ms_per_step=ms, gemv_us=gemv_ms * 1e3, gemv_GBps=gemv_bytes / (gemv_ms * 1e-3) / 1e9,
                            gemv_hbm_frac=gemv_bytes / (gemv_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                            gemv_b2b_us=b2b_ms * 1e3,
                            gemv_b2b_hbm_frac=gemv_bytes / (b2b_ms * 1e-3) / 1e9 / PEAK_HBM_GBS)
    return out


def bench_decode(torch, sq, d, wl, steps, warmup, copies=3):
    """M in {1,4,16} against 3 rotated copies of the int8 weight (705 MB > 256 MB MALL)."""
    W = wl.weights["w"]
    N, K = W.shape
    s, Wq0, ws = prepare_weight(torch, sq, d, wl.calib, W, wl.alpha, wl.gran)
    Wqs = [Wq0] + [Wq0.clone() for _ in range(copies - 1)]
    out = {}
    for M in wl.decode_rows:
        X = d(wl.X[:M])
        Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
        xs = torch.empty(M, dtype=torch.float32, device="cuda")
        Y = torch.empty(M, N, dtype=torch.float16, device="cuda")
        it = [0]

        def step(timer):
            Wq = Wqs[it[0] % copies]
            it[0] += 1
            sq.sq_quantize_per_token(X, s, Xq, xs)
            g = lambda: sq.w8a8_gemm_dequant(Xq, xs, Wq, ws, 0, None, Y)
            timer.around(g) if timer else g()

        # the step alone (no per-kernel events in the timed region), then the GEMV launches on their own:
        # each bracketed by events (dispatch included), and back to back (the stream's kernel rate)
        ms, _ = time_steps(torch, step, steps, warmup, kernel_events=False)
        _, gemv_ms = time_steps(torch, step, steps, 2)

        def gemv_only(timer):
            Wq = Wqs[it[0] % copies]
            it[0] += 1
            sq.w8a8_gemm_dequant(Xq, xs, Wq, ws, 0, None, Y)

        b2b_ms, _ = time_steps(torch, gemv_only, steps, 2, kernel_events=False)
        # warm cache: the same weight copy every step (it stays in the 256 MB MALL)
        warm_ms, _ = time_steps(torch, lambda t: (sq.sq_quantize_per_token(X, s, Xq, xs),
                                                  sq.w8a8_gemm_dequant(Xq, xs, Wq0, ws, 0, None, Y)),
                                steps, 2, kernel_events=False)
        # the same step as one call (M <= 4: quantization in the decode kernel's prologue)
        lws = torch.empty(sq.sq_workspace_size(sq.SQ_OP_LINEAR, M, N, K), dtype=torch.uint8, device="cuda")

        def linear(timer):
            Wq = Wqs[it[0] % copies]
            it[0] += 1
            sq.sq_w8a8_linear(X, s, Wq, ws, 0, None, Y, lws, xs)

        lin_ms, _ = time_steps(torch, linear, steps, 2, kernel_events=False)
        nbytes = N * K + 4 * N + 2 * M * K + 2 * M * K + 4 * M + 2 * M * N
        gemv_bytes = N * K + 4 * N + M * K + 4 * M + 2 * M * N
        out[f"M{M}"] = dict(ms_per_step=ms, GBps=nbytes / (ms * 1e-3) / 1e9,
                            hbm_frac=nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                            gemv_us=gemv_ms * 1e3,
                            gemv_GBps=gemv_bytes / (gemv_ms * 1e-3) / 1e9,
                            gemv_hbm_frac=gemv_bytes / (gemv_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                            gemv_b2b_us=b2b_ms * 1e3,
                            gemv_b2b_hbm_frac=gemv_bytes / (b2b_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                            warm_cache_step_us=warm_ms * 1e3,
                            linear_one_call_us=lin_ms * 1e3,
                            linear_one_call_hbm_frac=(N * K + 4 * N + 2 * M * K + 2 * M * N) / (lin_ms * 1e-3) / 1e9
                            / PEAK_HBM_GBS)
    out["gemv_traffic_bytes_per_launch"] = traffic_for("gemv_decode_70b", GEMV_SRC)
    return out


def bench_llm_int8(torch, sq, d, wl, steps, warmup):
    X, W16 = wl.X, wl.weights["w"]
    M, K = X.shape
    N = W16.shape[0]
    _, Wq, ws = prepare_weight(torch, sq, d, None, W16, None, 0)
    Xd, Wd = d(X), d(W16)
    Y = torch.empty(M, N, dtype=torch.float16, device="cuda")
    wsp = torch.empty(sq.sq_workspace_size(sq.SQ_OP_OUTLIER, M, N, K), dtype=torch.uint8, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step(timer):
        sq.int8_outlier_matmul(Xd, Wd, Wq, ws, None, wl.threshold, Y, wsp, cnt)

    settle(torch, step)
    ms, _ = time_steps(torch, step, steps, warmup)
    ops = 2.0 * M * N * K
    n_out = int(cnt.item())
    # the unquantized fp16 layer on the same operands, for the pages' LLM.int8() speed-up over fp16
    Yf = torch.empty(M, N, dtype=torch.float16, device="cuda")
    fp16_step = lambda _: torch.mm(Xd, Wd.t(), out=Yf)
    settle(torch, fp16_step, 0.3)
    fms, _ = time_steps(torch, fp16_step, steps, warmup, kernel_events=False)
    tflops = ops / (fms * 1e-3) / 1e12
    return dict(ms_per_step=ms, TOPS=ops / (ms * 1e-3) / 1e12, mfma_frac=ops / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS,
                n_outliers=n_out,
                fp16_reference=dict(ms_per_step=round(fms, 5), TFLOPs=round(tflops, 1),
                                    fp16_mfma_frac=round(tflops / PEAK_FP16_TFLOPS, 4),
                                    llm_int8_speedup=round(fms / ms, 3),
                                    call="torch.mm(X, W16.t(), out=Y), fp16 in and out"))


def bench_layernorm_quant(torch, sq, d, wl, steps, warmup):
    """LayerNorm with the smoothing folded into its weights, fused with per-token
    quantization, on the prefill activation (HBM-bound: 2 B read + 1 B written per
    element); the unfused smoothing + quantization step it replaces is timed beside it."""
    M, K = wl.X.shape
    X = d(wl.X)
    r = np.random.default_rng(3)
    g = d(r.uniform(0.5, 1.5, K).astype(np.float32))
    b = d((r.standard_normal(K) * 0.05).astype(np.float32))
    s = d(r.uniform(0.1, 10.0, K).astype(np.float32))
    g2, b2 = torch.empty_like(g), torch.empty_like(b)
    sq.sq_fold_smoothing_layernorm(g, b, s, g2, b2)
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")
    fused_ms, _ = time_steps(torch, lambda t: sq.sq_layernorm_quantize_per_token(X, g2, b2, 1e-5, Xq, xs),
                             steps, warmup, kernel_events=False)
    unfused_ms, _ = time_steps(torch, lambda t: sq.sq_quantize_per_token(X, s, Xq, xs), steps, warmup,
                               kernel_events=False)
    nbytes = 2 * M * K + M * K + 4 * M + 8 * K
    return dict(M=M, K=K, us=fused_ms * 1e3, GBps=nbytes / (fused_ms * 1e-3) / 1e9,
                hbm_frac=nbytes / (fused_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                smooth_quant_us=unfused_ms * 1e3)


def bench_static(torch, sq, d, wl_pre, wl_dec, steps, warmup, copies=3):
    """Static (calibrated, per-tensor) activation scale: quantization of the prefill
    activation and the decode step (quantize + GEMV) with it, each beside its
    per-token (dynamic) counterpart."""
    out = {}
    M, K = wl_pre.X.shape
    X = d(wl_pre.X)
    s = d(np.random.default_rng(5).uniform(0.1, 10.0, K).astype(np.float32))
    xs1 = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(sq.sq_workspace_size(sq.SQ_OP_CALIB_STATIC, M, 0, K), dtype=torch.uint8, device="cuda")
    sq.sq_calibrate_static_scale(X, s, 99.99, xs1, ws)
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    rows = torch.empty(M, dtype=torch.float32, device="cuda")
    ms, _ = time_steps(torch, lambda t: sq.sq_quantize_static(X, s, xs1, Xq, rows), steps, warmup, kernel_events=False)
    ms_dyn, _ = time_steps(torch, lambda t: sq.sq_quantize_per_token(X, s, Xq, rows), steps, warmup,
                           kernel_events=False)
    nbytes = 2 * M * K + M * K + 4 * M
    out["quantize_prefill"] = dict(M=M, K=K, us=ms * 1e3, GBps=nbytes / (ms * 1e-3) / 1e9,
                                   hbm_frac=nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, per_token_us=ms_dyn * 1e3)
    # decode: calibrated on the 512-token batch, three rotated weight copies
    W = wl_dec.weights["w"]
    N, K = W.shape
    sd, Wq0, wsc = prepare_weight(torch, sq, d, wl_dec.calib, W, wl_dec.alpha, wl_dec.gran)
    cal = d(wl_dec.calib)
    ws = torch.empty(sq.sq_workspace_size(sq.SQ_OP_CALIB_STATIC, cal.shape[0], 0, K), dtype=torch.uint8,
                     device="cuda")
    sq.sq_calibrate_static_scale(cal, sd, 99.99, xs1, ws)
    Wqs = [Wq0] + [Wq0.clone() for _ in range(copies - 1)]
    for Md in wl_dec.decode_rows:
        Xd = d(wl_dec.X[:Md])
        Xqd = torch.empty(Md, K, dtype=torch.int8, device="cuda")
        rowsd = torch.empty(Md, dtype=torch.float32, device="cuda")
        Y = torch.empty(Md, N, dtype=torch.float16, device="cuda")
        it = [0]

        def step(timer):
            Wq = Wqs[it[0] % copies]
            it[0] += 1
            sq.sq_quantize_static(Xd, sd, xs1, Xqd, rowsd)
            sq.w8a8_gemm_dequant(Xqd, rowsd, Wq, wsc, 0, None, Y)

        ms, _ = time_steps(torch, step, steps, warmup, kernel_events=False)
        nb = N * K + 4 * N + 2 * Md * K + 2 * Md * N
        out[f"decode_M{Md}"] = dict(ms_per_step=ms, GBps=nb / (ms * 1e-3) / 1e9,
                                    hbm_frac=nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS)
    return out


def bench_kv_cache(torch, sq, d, steps, warmup, copies=3, batch=16):
    """INT8 KV cache of one layer (8 KV heads x 128) for a batch of 16 sequences of
    4096 tokens: per-head calibration on a 512-token batch, quantization of K and V
    with the fixed scales, and the fp16 read-back.  Three rotated buffer sets keep
    the working set beyond the on-die caches."""
    import workloads
    K_cal, V_cal, Kx, Vx = workloads.kv_cache()
    T1, H, D = Kx.shape
    T = T1 * batch
    KV = [torch.cat([d(Kx)] * batch), torch.cat([d(Vx)] * batch)]
    sets = [[t.clone() for t in KV] for _ in range(copies)]
    sc = [torch.empty(H, dtype=torch.float32, device="cuda") for _ in range(2)]
    cal = [d(K_cal), d(V_cal)]
    for i in range(2):
        sq.sq_kv_calibrate_per_head(cal[i], 1.2, sc[i])
    ms_cal, _ = time_steps(torch, lambda t: sq.sq_kv_calibrate_per_head(cal[0], 1.2, sc[0]), steps, warmup,
                           kernel_events=False)
    q = [[torch.empty(T, H, D, dtype=torch.int8, device="cuda") for _ in range(2)] for _ in range(copies)]
    it = [0]

    def quant(timer):
        j = it[0] % copies
        it[0] += 1
        for i in range(2):
            sq.sq_kv_quantize_per_head(sets[j][i], sc[i], q[j][i])

    ms_q, _ = time_steps(torch, quant, steps, warmup, kernel_events=False)
    Y = [[torch.empty(T, H * D, dtype=torch.float16, device="cuda") for _ in range(2)] for _ in range(copies)]

    def deq(timer):
        j = it[0] % copies
        it[0] += 1
        for i in range(2):
            sq.sq_dequantize(q[j][i].view(T, H * D), sc[i], 0, D, Y[j][i])

    ms_d, _ = time_steps(torch, deq, steps, warmup, kernel_events=False)
    n = 2 * T * H * D
    qb, db = 3 * n + 8 * H, 3 * n + 8 * H
    return dict(tokens=T, heads=H, head_dim=D, calibrate_us=ms_cal * 1e3,
                quantize_kv=dict(us=ms_q * 1e3, GBps=qb / (ms_q * 1e-3) / 1e9,
                                 hbm_frac=qb / (ms_q * 1e-3) / 1e9 / PEAK_HBM_GBS),
                dequantize_kv=dict(us=ms_d * 1e3, GBps=db / (ms_d * 1e-3) / 1e9,
                                   hbm_frac=db / (ms_d * 1e-3) / 1e9 / PEAK_HBM_GBS))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_one_thread(wl, rows=16):
    """The oracle's forward path (quantize, int8 GEMM, dequant, store; LLM.int8()
    adds its outlier split and fp16 side product) on one thread, over the first
    `rows` token rows.  Weight preparation runs beforehand on every thread, untimed."""
    import oracle
    prepared = []
    for W in wl.weights.values():
        s = oracle.smooth_scales(wl.calib, W, wl.alpha)[1] if wl.alpha is not None else None
        prepared.append((W,) + (s,) + tuple(oracle.quantize_weight(W, s, wl.gran)))
    rows = min(rows, wl.X.shape[0])
    sel = np.arange(rows)
    n0 = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        t = time.perf_counter()
        for W, s, Wq, ws in prepared:
            if wl.threshold is not None:
                oracle.llm_int8_linear(wl.X, W, Wq, ws, wl.threshold, None, sel)
            else:
                oracle.w8a8_linear(wl.X[:rows], s, Wq, ws, wl.gran, None, wl.out_dtype)
        t = time.perf_counter() - t
    finally:
        oracle.set_num_threads(n0)
    ops = sum(2.0 * rows * W.shape[0] * W.shape[1] for W in wl.weights.values())
    return dict(rows=rows, seconds=round(t, 3), GOPs=round(ops / t / 1e9, 3))


def cpu_baseline(wl, target_s):
    """The oracle on the same per-token work (quantize + int8 GEMM + dequant +
    fp16 store, every projection) for a bounded number of token rows."""
    import oracle
    import workloads
    prepared = []
    for name, W in wl.weights.items():
        s = oracle.smooth_scales(wl.calib, W, wl.alpha)[1] if wl.alpha is not None else None
        Wq, ws = oracle.quantize_weight(W, s, wl.gran)
        prepared.append((s, Wq, ws))

    def run(rows):
        t = time.perf_counter()
        for s, Wq, ws in prepared:
            oracle.w8a8_linear(wl.X[:rows], s, Wq, ws, wl.gran, None, wl.out_dtype)
        return time.perf_counter() - t

    r0 = 8
    t0 = run(r0)
    rows = int(min(wl.X.shape[0], max(r0, round(r0 * target_s / max(t0, 1e-6)))))
    t = run(rows)
    K = wl.X.shape[1]
    ops = sum(2.0 * rows * W.shape[0] * K for W in wl.weights.values())
    return dict(value=ops / t / 1e12, unit="TOPS", cores=oracle.num_threads(), kind="oracle",
                sample=f"first {rows} of {wl.X.shape[0]} token rows, all {len(wl.weights)} projections "
                       f"({ops / 1e9:.1f} GOP in {t:.1f} s)",
                cpu_model=cpu_model(),
                one_thread={"single_w8a8_16x512x512": oracle_one_thread(workloads.single_w8a8()),
                            wl.name + "_16_rows": oracle_one_thread(wl)})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10,
                    help="untimed steps before the timed ones (after the clock-settle phase)")
    ap.add_argument("--quick", action="store_true", help="headline workload (the 530B slice) only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", default=None,
                    help="run one workload: slice_530b|prefill_7b|decode_70b|llm_int8|zero_point|layernorm_quant|static_quant|kv_cache|fp8")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer runs on a single MI355X).", flush=True)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": a.numel() * 4, "launches": 5}))
        return

    import int8_quantization_amd as sq
    import workloads

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    result = {}
    secondary = {}
    if args.only in (None, "slice_530b"):
        log("slice_530b: generating inputs")
        wl = workloads.slice_530b()
        log("slice_530b: timing")
        r = bench_w8a8(torch, sq, d, wl, args.steps, args.warmup)
        M, K, N = wl.M, wl.K, r["Ns"][0]
        tops = r["ops"] / (r["ms"] * 1e-3) / 1e12
        gemm_tops = r["gemm_ops_per_launch"] / (r["gemm_ms"] * 1e-3) / 1e12
        traffic = traffic_for("gemm_slice_530b", GEMM_SRC)
        result = {
            "metric": METRIC, "value": round(tops, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(r["ms"], 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "int8", "data": "synthetic",
            "config": {"workload": wl.name, "M": M, "K": K, "N": N, "alpha": wl.alpha,
                       "weight_scale": "per_tensor", "act_scale": "per_token", "out_dtype": "fp16",
                       "parallelism": "single_gpu"},
            "mfma_frac_incl_quant": round(tops / PEAK_INT8_TOPS, 4),
            "clock_settle_steps": r["settle_steps"],
            "step_ms_percentiles": {k: round(v, 5) for k, v in r["pct"].items()},
            "tops_at_p50": round(r["ops"] / (r["pct"]["p50"] * 1e-3) / 1e12, 2),
            "quantize_530b": r["quantize"],
            "fp16_reference": r["fp16_reference"],
            "gpu": gpu_info(torch),
            "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                         "frac": round(gemm_tops / PEAK_INT8_TOPS, 4), "traffic": traffic,
                         "kernel": "gemm_i8_kernel (int8 MFMA GEMM + dequant epilogue), two launches per call",
                         "launches": [
                             {"tiles": "256x256", "output_columns": [0, 8192], "tile_count": 512,
                              "algorithmic_ops": 2.0 * M * 8192 * K},
                             {"tiles": "128x128", "output_columns": [8192, N], "tile_count": 512,
                              "algorithmic_ops": 2.0 * M * (N - 8192) * K}],
                         "gemm_us_per_call": round(r["gemm_ms"] * 1e3, 2),
                         "algorithmic_ops_per_call": r["gemm_ops_per_launch"]},
        }
        if not args.no_cpu_baseline:
            log("slice_530b: CPU oracle baseline")
            result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        del wl, r
        torch.cuda.empty_cache()
    if not args.quick:
        sec_steps, sec_warm = max(5, args.steps // 2), max(2, args.warmup // 2)
        if args.only in (None, "prefill_7b"):
            log("prefill_7b: generating inputs")
            wl2 = workloads.prefill_7b()
            r = bench_w8a8(torch, sq, d, wl2, sec_steps * 2, sec_warm)
            gemm_tops = r["gemm_ops_per_launch"] / (r["gemm_ms"] * 1e-3) / 1e12
            tops = r["ops"] / (r["ms"] * 1e-3) / 1e12
            secondary["prefill_7b"] = dict(
                workload=wl2.name, ms_per_step=r["ms"], TOPS=tops, mfma_frac_incl_quant=tops / PEAK_INT8_TOPS,
                step_ms_percentiles=r["pct"], gemm_us_per_launch=r["gemm_ms"] * 1e3, gemm_TOPS=gemm_tops,
                gemm_mfma_frac=gemm_tops / PEAK_INT8_TOPS, quantize_7b=r["quantize"],
                gemm_traffic_bytes_per_launch=traffic_for("gemm_prefill_7b", GEMM_SRC),
                fp16_reference=r["fp16_reference"])
            if not args.no_cpu_baseline:
                secondary["prefill_7b"]["cpu_oracle_one_thread"] = oracle_one_thread(wl2)
            del wl2
            torch.cuda.empty_cache()
        if args.only in (None, "decode_70b"):
            log("decode_70b: generating inputs")
            wl3 = workloads.decode_70b()
            secondary["decode_70b"] = bench_decode(torch, sq, d, wl3, sec_steps * 2, sec_warm)
            if not args.no_cpu_baseline:
                secondary["decode_70b"]["cpu_oracle_one_thread"] = oracle_one_thread(wl3)
            del wl3
        if args.only in (None, "llm_int8"):
            log("llm_int8: generating inputs")
            wl4 = workloads.llm_int8_4096()
            secondary["llm_int8"] = bench_llm_int8(torch, sq, d, wl4, sec_steps, sec_warm)
            if not args.no_cpu_baseline:
                secondary["llm_int8"]["cpu_oracle_one_thread"] = oracle_one_thread(wl4)
            del wl4
        if args.only in (None, "zero_point"):
            log("zero_point: generating inputs")
            wl5 = workloads.ffn_down_7b_post_activation()
            secondary["zero_point_ffn_down_7b"] = bench_zero_point(torch, sq, d, wl5, sec_steps * 2, sec_warm)
            del wl5
            torch.cuda.empty_cache()
        if args.only in (None, "layernorm_quant"):
            log("layernorm_quant: prefill activation")
            secondary["layernorm_quant_7b"] = bench_layernorm_quant(torch, sq, d, workloads.prefill_7b(which=("qkv",)),
                                                                    sec_steps * 4, sec_warm)
        if args.only in (None, "static_quant"):
            log("static_quant: prefill activation and decode")
            secondary["static_scale"] = bench_static(torch, sq, d, workloads.prefill_7b(which=("qkv",)),
                                                     workloads.decode_70b(), sec_steps * 2, sec_warm)
        if args.only in (None, "fp8"):
            log("fp8: 7B prefill projections with FP8 E4M3 codes")
            secondary["fp8_prefill_7b"] = bench_fp8(torch, sq, d, workloads.prefill_7b(), sec_steps, sec_warm)
            torch.cuda.empty_cache()
            secondary["fp8_decode_70b"] = bench_fp8_decode(torch, sq, d, workloads.decode_70b(), sec_steps * 2,
                                                           sec_warm)
            torch.cuda.empty_cache()
        if args.only in (None, "kv_cache"):
            log("kv_cache: 16 x 4096 tokens, 8 heads x 128")
            secondary["kv_cache"] = bench_kv_cache(torch, sq, d, sec_steps * 2, sec_warm)
            torch.cuda.empty_cache()
        torch.cuda.empty_cache()
        result["secondary"] = secondary
    if not result.get("metric"):
        result = {"metric": METRIC, "value": None, "secondary": secondary}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
