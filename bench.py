#!/usr/bin/env python3
"""Benchmark of the NVFP4 linear-layer hot path on one MI355X.

One step = one pass over one batch of the NVFP4 workload with 4096 tokens,
hidden 2048 and 768 outputs (the second configuration of the benchmark set):
  1. per-token NVFP4 quantization of the activations X [4096, 2048]
  2. 16x16 NVFP4 quantization of the weight W [768, 2048] (per-tensor scale:
     an amax pass, then the quantize pass, which also writes the dequantized
     BF16 copy DQ(Q(W)) [768, 2048], the dequantized-backward operand)
  3. FPROP  Y [4096, 768]  = Q(X) Q(W)^T       (NVFP4 x NVFP4, BF16 out)
  4. DGRAD dX [4096, 2048] = dY DQ(Q(W))       (BF16, weight read transposed)
Inputs are seeded synthetic tensors (the pages' models and datasets stand in
as shapes and distributions only), resident in HBM before timing; ten
buffer sets (> 512 MB in total) rotate so reads come from HBM rather than
the 256 MB last-level cache.

Prints ONE JSON line on stdout.  `value` is the step's GEMM throughput: the
two GEMMs' algorithmic flops (2*M*N*K each) over the whole step's time,
quantization and dequantization included.  The step is timed two ways, both
reported: plain launches back to back on one stream, and replays of the step
captured once per buffer set as a HIP graph (the library records no memsets,
so every node is a kernel); `value` takes the faster and `launch` names it.
`--overlap` forks the weight path (Q(W) with DQ(W)), which depends on no
activation, to a second stream inside the graph; on MI355X that measured
slower.  `--eager` skips the graph.  Per-stage times (HIP events around each
stage of spin-fronted eager steps), GB/s, TFLOP/s and fractions of peak are
in "kernels"; "roofline" times the stage with the largest share again over
runs of back-to-back launches.  The CPU oracle, timed on a bounded sample of
the same step, is reported as "cpu_baseline".
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

M, K, N = 4096, 2048, 768
PEAK_HBM_GBPS = 8000.0
PEAK_F16_TFLOPS = 2500.0     # dense FP16/BF16 MFMA
PEAK_FP4_TFLOPS = 10100.0    # dense FP4 MFMA (context for the NVFP4 GEMM)
SETS = 10

# algorithmic bytes / flops per launch
BYTES_QX = M * K * 2 + M * K // 2 + M * (K // 16) + M * 4
# Q(W) and DQ(W) in one pass: two reads of W (amax, quantize), codes, scales,
# S and the BF16 dequantized copy
BYTES_QDQW = 2 * N * K * 2 + N * K // 2 + (N // 16) * (K // 16) + 4 + N * K * 2
FLOPS_FPROP = 2 * M * N * K
FLOPS_DGRAD = 2 * M * K * N


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


COPY_BYTES = 256 << 20
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "microscaling_quantization_block_amd", "csrc", "gemm.hip")


def measured_reference(m, torch):
    """Context for the spec peaks: the bandwidth of a plain device copy of
    COPY_BYTES (read + write bytes over time, HIP events, 20 copies), and the
    host cost of one library call from Python (binding + C ABI + launch,
    2000 back-to-back calls of a 64x64 MXFP8 dequantize, no synchronization)."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(20):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * COPY_BYTES * 20 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    x = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    c, s = m.mx_quantize(x)
    out = torch.empty_like(x)
    for _ in range(50):
        m.mx_dequantize(m.Format.MXFP8, c, s, 64, 64, out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(2000):
        m.mx_dequantize(m.Format.MXFP8, c, s, 64, 64, out=out)
    host_us = (time.perf_counter() - t0) / 2000 * 1e6
    torch.cuda.synchronize()
    return {"copy_GBps": round(copy_gbps, 1), "copy_frac_of_hbm_peak": round(copy_gbps / PEAK_HBM_GBPS, 4),
            "host_us_per_call": round(host_us, 2),
            "note": "device copy of 256 MiB (read + write bytes); host time of one Python -> C ABI call"}


def copy_calibration():
    """A plain device copy of COPY_BYTES, ten times: the reference for scaling
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 10}), flush=True)


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter record, or
    None when there is none or the GEMM source changed since it was taken."""
    try:
        rec = json.load(open(TRAFFIC_RECORD))
        sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel") != kernel or rec.get("gemm_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def make_sets(m, torch, data):
    import numpy as np
    dev = "cuda"

    def bf(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)

    x0, w0, dy0 = bf(data["x"]), bf(data["w"]), bf(data["dy"])
    sets = []
    for _ in range(SETS):
        s = dict(x=x0.clone(), w=w0.clone(), dy=dy0.clone())
        s["cx"] = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        s["sx"] = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
        s["Sx"] = torch.empty(M, dtype=torch.float32, device=dev)
        s["cw"] = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        s["sw"] = torch.empty((N // 16, K // 16), dtype=torch.uint8, device=dev)
        s["Sw"] = torch.empty(1, dtype=torch.float32, device=dev)
        s["y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        s["wdq"] = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        s["dx"] = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        sets.append(s)
    return sets


def step_concurrent(m, s, side, torch):
    """The same stages with the weight path (Q(W) with DQ(W)) on a second
    stream beside Q(X); FPROP waits for it."""
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        m.nvfp4_quantize_dq(s["w"], codes=s["cw"], block_scales=s["sw"], gscales=s["Sw"], dq=s["wdq"])
        qw_done = torch.cuda.Event()
        qw_done.record(side)
    m.nvfp4_quantize(s["x"], gs=m.GScale.PER_ROW, codes=s["cx"], block_scales=s["sx"], gscales=s["Sx"])
    main.wait_event(qw_done)
    m.mx_gemm(m.Operand(m.Format.NVFP4, s["cx"], s["sx"], s["Sx"], gs=m.GScale.PER_ROW),
              m.Operand(m.Format.NVFP4, s["cw"], s["sw"], s["Sw"], block=m.Block.TILE,
                        gs=m.GScale.PER_TENSOR), M, N, K, out=s["y"])
    main.wait_stream(side)
    m.mx_gemm(m.Operand(m.Format.BF16, s["dy"], block=m.Block.NONE),
              m.Operand(m.Format.BF16, s["wdq"], block=m.Block.NONE, transposed=True), M, K, N,
              out=s["dx"])


def stages(m):
    """The four stages of the step, each a function of one buffer set: per-token
    Q(X); 16x16 Q(W) with its dequantized copy DQ(W) written in the same pass;
    FPROP; dequantized-backward DGRAD."""
    def qx(s):
        m.nvfp4_quantize(s["x"], gs=m.GScale.PER_ROW, codes=s["cx"], block_scales=s["sx"], gscales=s["Sx"])

    def qdqw(s):
        m.nvfp4_quantize_dq(s["w"], codes=s["cw"], block_scales=s["sw"], gscales=s["Sw"], dq=s["wdq"])

    def fprop(s):
        m.mx_gemm(m.Operand(m.Format.NVFP4, s["cx"], s["sx"], s["Sx"], gs=m.GScale.PER_ROW),
                  m.Operand(m.Format.NVFP4, s["cw"], s["sw"], s["Sw"], block=m.Block.TILE,
                            gs=m.GScale.PER_TENSOR), M, N, K, out=s["y"])

    def dgrad(s):
        m.mx_gemm(m.Operand(m.Format.BF16, s["dy"], block=m.Block.NONE),
                  m.Operand(m.Format.BF16, s["wdq"], block=m.Block.NONE, transposed=True), M, K, N,
                  out=s["dx"])
    return [qx, qdqw, fprop, dgrad]


def step(m, s, ev=None):
    """One step: the four stages in order.  ev (list of 5 events) brackets
    each stage if given."""
    for i, fn in enumerate(stages(m)):
        if ev is not None:
            ev[i].record()
        fn(s)
    if ev is not None:
        ev[4].record()


def batch_us(torch, fn, sets, spin, repeats):
    """Mean time of one launch of `fn` over back-to-back launches on every
    buffer set in turn: HIP events around each run of len(sets) launches,
    each run behind a spin kernel so that the launches are all queued before
    the first event fires."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(repeats)]
    torch.cuda.synchronize()
    for a, b in evs:
        torch.cuda._sleep(spin)
        a.record()
        for s_ in sets:
            fn(s_)
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / (repeats * len(sets)) * 1e3


SPIN_US = 100.0        # longer than the host takes to enqueue one step
BATCH_SPIN_US = 300.0  # longer than it takes to enqueue one launch per buffer set


def spin_cycles(torch, us):
    """Argument of torch.cuda._sleep (a one-thread spin on the GPU clock
    counter) that spins for about `us` microseconds, from one timed probe."""
    probe = 1 << 20
    torch.cuda._sleep(probe)                      # first launch outside the probe
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    torch.cuda._sleep(probe)
    b.record()
    torch.cuda.synchronize()
    per_us = probe / max(a.elapsed_time(b) * 1e3, 1.0)
    return max(int(per_us * us), 1)


def cpu_baseline(data, min_seconds):
    """The oracle, as it stands, on the same step: the full step (all tokens)
    repeated until at least `min_seconds` of CPU time have passed; the sample
    is bounded by that time."""
    import numpy as np
    from oracle import formats as F, nvfp4 as ON, gemm as G
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = len(os.sched_getaffinity(0))
    xv = F.bf16_bits_to_f64(data["x"])
    wv = F.bf16_bits_to_f64(data["w"])
    dyv = F.bf16_bits_to_f64(data["dy"])
    reps = 0
    t0 = time.perf_counter()
    while True:
        wc, wsb, wS = ON.quantize_tile16(wv)
        w64 = ON.dequantize_f64(wc, wsb, wS, "16x16", "per_tensor")
        wdq = ON.dequantize_bf16(wc, wsb, wS, "16x16", "per_tensor")
        xc, xsb, xS = ON.quantize_rowwise(xv, "per_row")
        x64 = ON.dequantize_f64(xc, xsb, xS, "1x16", "per_row")
        y = F.bf16_rne(G.gemm_f64(x64, w64))
        dx = F.bf16_rne(G.gemm_f64(dyv, F.bf16_bits_to_f64(wdq).T.copy()))
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    t_step = el / reps
    assert y.shape == (M, N) and dx.shape == (M, K)
    return dict(value=(FLOPS_FPROP + FLOPS_DGRAD) / t_step / 1e12, unit="TFLOP/s",
                cores=int(blas_threads), kind="oracle",
                sample=(f"the full step ({M} tokens: Q(X), 16x16 Q(W), DQ(W), FPROP and DGRAD "
                        f"as float64 dequantize-then-matmul) repeated {reps} times in {el:.1f} s; "
                        f"quantizers single-threaded NumPy, matmuls on {blas_threads} BLAS threads"),
                seconds_per_step=round(t_step, 3))


# ---------------------------------------------------------------- --rows
PEAK_FP8_TFLOPS = 5000.0


def _time_us(torch, fn, iters, warm_ms=30.0):
    # warm up until about warm_ms of work has run (at least three calls): the
    # clock drops while the host sets up a row, and a cold start reads slow
    t0, n = time.perf_counter(), 0
    while n < 3 or (time.perf_counter() - t0) * 1e3 < warm_ms:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters * 1e3


def rows_report():
    """Each hot-path row at the other configurations' shapes: quantizers and
    dequantizers against HBM bandwidth, GEMMs against their dtype's MFMA
    peak, the MoE stages of the Qwen3-30B-A3B-shaped layer.  One JSON line
    per measurement (HIP events around repeated launches, inputs resident)."""
    import numpy as np
    import torch
    import microscaling_quantization_block_amd as m
    import synth
    dev = "cuda"

    def out(row, what, shape, us, nbytes=None, flops=None, peak=None, fp4=False):
        d = dict(row=row, what=what, shape=shape, us=round(us, 2))
        if nbytes is not None:
            gbps = nbytes / (us * 1e-6) / 1e9
            d.update(bytes=int(nbytes), GBps=round(gbps, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                     frac=round(gbps / PEAK_HBM_GBPS, 4), bound="hbm")
        else:
            tf = flops / (us * 1e-6) / 1e12
            d.update(flops=int(flops), TFLOPs=round(tf, 1), peak=peak, unit="TFLOP/s",
                     frac=round(tf / peak, 4), bound="mfma")
            if fp4:
                d["frac_fp4_peak"] = round(tf / PEAK_FP4_TFLOPS, 4)
        print(json.dumps(d), flush=True)

    # ---- Llama-3-8B-shaped dense MLP, NVFP4 (tokens 32768, hidden 4096, I 14336)
    T5, H5, I5 = 32768, 4096, 14336
    x5 = synth.torch_normal_bf16((T5, H5), 1.0, 51, dev)
    n = T5 * H5
    cx, sx, Sx = m.nvfp4_quantize(x5)
    out("a1-a3", "nvfp4 1x16 per-token RNE (X)", [T5, H5], _time_us(torch, lambda: m.nvfp4_quantize(
        x5, codes=cx, block_scales=sx, gscales=Sx), 10), nbytes=n * 2 + n // 2 + n // 16 + T5 * 4)
    out("f2", "nvfp4 1x16 per-token RNE + Four-Over-Six (X)", [T5, H5], _time_us(torch, lambda: m.nvfp4_quantize(
        x5, rnd=m.Round.RNE_4OVER6, codes=cx, block_scales=sx, gscales=Sx), 10),
        nbytes=n * 2 + n // 2 + n // 16 + T5 * 4)
    dy5 = synth.torch_normal_bf16((T5, H5), 1e-3, 52, dev)          # down-projection output gradient
    cg, sg, Sg = m.nvfp4_quantize(dy5, rnd=m.Round.SR)
    out("a1-a3", "nvfp4 1x16 per-token SR (dY)", [T5, H5], _time_us(torch, lambda: m.nvfp4_quantize(
        dy5, rnd=m.Round.SR, codes=cg, block_scales=sg, gscales=Sg), 10), nbytes=n * 2 + n // 2 + n // 16 + T5 * 4)
    cgc, sgc, Sgc = m.nvfp4_quantize(dy5, block=m.Block.COL, gs=m.GScale.PER_TENSOR, rnd=m.Round.SR, stream_id=1)
    out("a1-a3", "nvfp4 16x1 columnwise per-tensor SR (dY^T, WGRAD)", [T5, H5], _time_us(torch, lambda: m.nvfp4_quantize(
        dy5, block=m.Block.COL, gs=m.GScale.PER_TENSOR, rnd=m.Round.SR, stream_id=1, codes=cgc,
        block_scales=sgc, gscales=Sgc), 10), nbytes=2 * n * 2 + n // 2 + n // 16 + 4)
    # the WGRAD inputs under the random Hadamard transform (two passes, both transforming)
    out("f1", "nvfp4 16x1 columnwise + RHT per-tensor SR (dY^T, WGRAD)", [T5, H5], _time_us(
        torch, lambda: m.nvfp4_quantize_rht(dy5, 0x6B2D, rnd=m.Round.SR, codes=cgc, block_scales=sgc,
                                            gscales=Sgc), 10), nbytes=2 * n * 2 + n // 2 + n // 16 + 4)
    out("f1", "nvfp4 16x1 columnwise + RHT per-tensor RNE (X^T, WGRAD)", [T5, H5], _time_us(
        torch, lambda: m.nvfp4_quantize_rht(x5, 0x6B2D, codes=cgc, block_scales=sgc, gscales=Sgc), 10),
        nbytes=2 * n * 2 + n // 2 + n // 16 + 4)
    out("a1-a3", "nvfp4 16x1 columnwise per-tensor RNE (X^T, WGRAD)", [T5, H5], _time_us(
        torch, lambda: m.nvfp4_quantize(x5, block=m.Block.COL, gs=m.GScale.PER_TENSOR, codes=cgc,
                                        block_scales=sgc, gscales=Sgc), 10),
        nbytes=2 * n * 2 + n // 2 + n // 16 + 4)
    w5 = synth.torch_normal_bf16((2 * I5, H5), 0.02, 53, dev)       # gate_up weight [N, K]
    nw = w5.numel()
    cw, sw, Sw = m.nvfp4_quantize(w5, block=m.Block.TILE, gs=m.GScale.PER_TENSOR)
    out("a1-a3", "nvfp4 16x16 per-tensor (W_gate_up)", [2 * I5, H5], _time_us(torch, lambda: m.nvfp4_quantize(
        w5, block=m.Block.TILE, gs=m.GScale.PER_TENSOR, codes=cw, block_scales=sw, gscales=Sw), 10),
        nbytes=2 * nw * 2 + nw // 2 + nw // 256 + 4)
    out("f2", "nvfp4 16x16 per-tensor + Four-Over-Six (W_gate_up)", [2 * I5, H5], _time_us(
        torch, lambda: m.nvfp4_quantize(w5, block=m.Block.TILE, gs=m.GScale.PER_TENSOR,
                                        rnd=m.Round.RNE_4OVER6, codes=cw, block_scales=sw, gscales=Sw), 10),
        nbytes=2 * nw * 2 + nw // 2 + nw // 256 + 4)
    wdq = torch.empty_like(w5)
    out("a4", "nvfp4 dequantize 16x16 -> bf16 (W_gate_up)", [2 * I5, H5], _time_us(torch, lambda: m.mx_dequantize(
        m.Format.NVFP4, cw, sw, 2 * I5, H5, block=m.Block.TILE, gscales=Sw, gs=m.GScale.PER_TENSOR, out=wdq), 10),
        nbytes=nw // 2 + nw // 256 + 4 + nw * 2)
    y5 = torch.empty((T5, 2 * I5), dtype=torch.bfloat16, device=dev)
    f = 2.0 * T5 * 2 * I5 * H5
    A = m.Operand(m.Format.NVFP4, cx, sx, Sx, gs=m.GScale.PER_ROW)
    B = m.Operand(m.Format.NVFP4, cw, sw, Sw, block=m.Block.TILE, gs=m.GScale.PER_TENSOR)
    out("a6", "nvfp4 FPROP gate_up", [T5, 2 * I5, H5], _time_us(torch, lambda: m.mx_gemm(A, B, T5, 2 * I5, H5, out=y5), 3),
        flops=f, peak=PEAK_F16_TFLOPS, fp4=True)
    del y5, wdq
    dyg = synth.torch_normal_bf16((T5, 2 * I5), 1e-3, 54, dev)       # gate_up output gradient
    cdg, sdg, Sdg = m.nvfp4_quantize(dyg, rnd=m.Round.SR)
    dx5 = torch.empty((T5, H5), dtype=torch.bfloat16, device=dev)
    Bt = m.Operand(m.Format.NVFP4, cw, sw, Sw, block=m.Block.TILE, gs=m.GScale.PER_TENSOR, transposed=True)
    Ad = m.Operand(m.Format.NVFP4, cdg, sdg, Sdg, gs=m.GScale.PER_ROW)
    out("a6", "nvfp4 DGRAD gate_up (16x16 weight read transposed)", [T5, H5, 2 * I5],
        _time_us(torch, lambda: m.mx_gemm(Ad, Bt, T5, H5, 2 * I5, out=dx5), 3), flops=f, peak=PEAK_F16_TFLOPS, fp4=True)
    ccg, scg, Scg = m.nvfp4_quantize(dyg, block=m.Block.COL, gs=m.GScale.PER_TENSOR, rnd=m.Round.SR, stream_id=1)
    ccx, scx, Scx = m.nvfp4_quantize(x5, block=m.Block.COL, gs=m.GScale.PER_TENSOR)
    dw = torch.empty((2 * I5, H5), dtype=torch.bfloat16, device=dev)
    Ag = m.Operand(m.Format.NVFP4, ccg, scg, Scg, gs=m.GScale.PER_TENSOR)
    Bx = m.Operand(m.Format.NVFP4, ccx, scx, Scx, gs=m.GScale.PER_TENSOR)
    out("a6", "nvfp4 WGRAD gate_up (columnwise copies)", [2 * I5, H5, T5],
        _time_us(torch, lambda: m.mx_gemm(Ag, Bx, 2 * I5, H5, T5, out=dw), 3), flops=f, peak=PEAK_F16_TFLOPS, fp4=True)
    del x5, dy5, w5, dyg, cdg, ccg, dx5, dw, cx, cg, cgc, cw, ccx
    torch.cuda.empty_cache()

    # ---- Qwen3-8B-shaped dense MLP, MXFP8 (tokens 8192, hidden 4096, I 12288)
    T4, H4, I4 = 8192, 4096, 12288
    x4 = synth.torch_normal_bf16((T4, H4), 1.0, 41, dev)
    n = T4 * H4
    mc, ms = m.mx_quantize(x4)
    out("a1-a3", "mxfp8 1x32 (X)", [T4, H4], _time_us(torch, lambda: m.mx_quantize(x4, codes=mc, scales=ms), 10),
        nbytes=n * 2 + n + n // 32)
    d4 = m.mx_quantize(x4, block=m.Block.DUAL)
    out("a1-a3", "mxfp8 dual rowwise + columnwise (X)", [T4, H4], _time_us(torch, lambda: m.mx_quantize(
        x4, block=m.Block.DUAL, codes=d4[0], scales=d4[1], codes_col=d4[2], scales_col=d4[3]), 10),
        nbytes=n * 2 + 2 * n + 2 * (n // 32))
    w4 = synth.torch_normal_bf16((2 * I4, H4), 0.02, 43, dev)
    nw = w4.numel()
    wc, wsc = m.mx_quantize(w4, block=m.Block.TILE)
    out("a1-a3", "mxfp8 32x32 (W_gate_up)", [2 * I4, H4], _time_us(torch, lambda: m.mx_quantize(
        w4, block=m.Block.TILE, codes=wc, scales=wsc), 10), nbytes=nw * 2 + nw + nw // 1024)
    wt4 = m.mx_quantize(w4, block=m.Block.TILE, transposed_copy=True)
    out("a1-a3", "mxfp8 32x32 + transposed copy (W_gate_up)", [2 * I4, H4], _time_us(torch, lambda: m.mx_quantize(
        w4, block=m.Block.TILE, codes=wt4[0], scales=wt4[1], codes_col=wt4[2], scales_col=wt4[3],
        transposed_copy=True), 10), nbytes=nw * 2 + 2 * nw + 2 * (nw // 1024))
    xo = torch.empty_like(x4)
    out("a4", "mxfp8 dequantize 1x32 -> bf16 (X)", [T4, H4], _time_us(torch, lambda: m.mx_dequantize(
        m.Format.MXFP8, mc, ms, T4, H4, out=xo), 10), nbytes=n + n // 32 + n * 2)
    y4 = torch.empty((T4, 2 * I4), dtype=torch.bfloat16, device=dev)
    f = 2.0 * T4 * 2 * I4 * H4
    A = m.Operand(m.Format.MXFP8, mc, ms)
    B = m.Operand(m.Format.MXFP8, wc, wsc, block=m.Block.TILE)
    out("a5", "mxfp8 FPROP gate_up", [T4, 2 * I4, H4], _time_us(torch, lambda: m.mx_gemm(A, B, T4, 2 * I4, H4, out=y4), 5),
        flops=f, peak=PEAK_FP8_TFLOPS)
    dyg4 = synth.torch_normal_bf16((T4, 2 * I4), 1e-3, 44, dev)
    dd = m.mx_quantize(dyg4, block=m.Block.DUAL)
    dx4 = torch.empty((T4, H4), dtype=torch.bfloat16, device=dev)
    out("a5", "mxfp8 DGRAD gate_up (32x32 weight read transposed)", [T4, H4, 2 * I4], _time_us(torch, lambda: m.mx_gemm(
        m.Operand(m.Format.MXFP8, dd[0], dd[1]), m.Operand(m.Format.MXFP8, wc, wsc, block=m.Block.TILE, transposed=True),
        T4, H4, 2 * I4, out=dx4), 5), flops=f, peak=PEAK_FP8_TFLOPS)
    out("a5", "mxfp8 DGRAD gate_up (transposed 32x32 copy)", [T4, H4, 2 * I4], _time_us(torch, lambda: m.mx_gemm(
        m.Operand(m.Format.MXFP8, dd[0], dd[1]), m.Operand(m.Format.MXFP8, wt4[2], wt4[3], block=m.Block.TILE),
        T4, H4, 2 * I4, out=dx4), 5), flops=f, peak=PEAK_FP8_TFLOPS)
    dw4 = torch.empty((2 * I4, H4), dtype=torch.bfloat16, device=dev)
    out("a5", "mxfp8 WGRAD gate_up (columnwise copies)", [2 * I4, H4, T4], _time_us(torch, lambda: m.mx_gemm(
        m.Operand(m.Format.MXFP8, dd[2], dd[3]), m.Operand(m.Format.MXFP8, d4[2], d4[3]), 2 * I4, H4, T4, out=dw4), 5),
        flops=f, peak=PEAK_FP8_TFLOPS)
    # the same layer with DeepSeek-style blockwise FP8 (1x128 / 128x128, power-of-two scales)
    b4 = m.fp8bw_quantize(x4, block=m.Block.DUAL)
    out("f4", "fp8 blockwise dual 1x128 + 128x1 (X)", [T4, H4], _time_us(torch, lambda: m.fp8bw_quantize(
        x4, block=m.Block.DUAL, codes=b4[0], scales=b4[1], codes_col=b4[2], scales_col=b4[3]), 10),
        nbytes=n * 2 + 2 * n + 2 * (n // 128))
    bw4 = m.fp8bw_quantize(w4, block=m.Block.TILE, transposed_copy=True)
    out("f4", "fp8 blockwise 128x128 + transposed copy (W_gate_up)", [2 * I4, H4], _time_us(
        torch, lambda: m.fp8bw_quantize(w4, block=m.Block.TILE, codes=bw4[0], scales=bw4[1], codes_col=bw4[2],
                                        scales_col=bw4[3], transposed_copy=True), 10),
        nbytes=nw * 2 + 2 * nw + 2 * (nw // 16384))
    bd = m.fp8bw_quantize(dyg4, block=m.Block.DUAL)
    F8 = m.Format.FP8_B128
    out("f4", "fp8 blockwise FPROP gate_up", [T4, 2 * I4, H4], _time_us(torch, lambda: m.mx_gemm(
        m.Operand(F8, b4[0], b4[1]), m.Operand(F8, bw4[0], bw4[1], block=m.Block.TILE), T4, 2 * I4, H4, out=y4), 5),
        flops=f, peak=PEAK_FP8_TFLOPS)
    out("f4", "fp8 blockwise DGRAD gate_up (transposed 128x128 copy)", [T4, H4, 2 * I4], _time_us(
        torch, lambda: m.mx_gemm(m.Operand(F8, bd[0], bd[1]), m.Operand(F8, bw4[2], bw4[3], block=m.Block.TILE),
                                 T4, H4, 2 * I4, out=dx4), 5), flops=f, peak=PEAK_FP8_TFLOPS)
    out("f4", "fp8 blockwise WGRAD gate_up (columnwise copies)", [2 * I4, H4, T4], _time_us(
        torch, lambda: m.mx_gemm(m.Operand(F8, bd[2], bd[3]), m.Operand(F8, b4[2], b4[3]), 2 * I4, H4, T4, out=dw4),
        5), flops=f, peak=PEAK_FP8_TFLOPS)
    # and with binary32 block scales (the partial sums of each 128-K block
    # scaled outside the MFMA, in a kernel of its own)
    del bd
    f4 = m.fp8bw_quantize_f32(x4, block=m.Block.DUAL)
    out("f4", "fp8 blockwise f32-scale dual 1x128 + 128x1 (X)", [T4, H4], _time_us(torch, lambda: m.fp8bw_quantize_f32(
        x4, block=m.Block.DUAL, codes=f4[0], scales=f4[1], codes_col=f4[2], scales_col=f4[3]), 10),
        nbytes=n * 2 + 2 * n + 8 * (n // 128))
    fw4 = m.fp8bw_quantize_f32(w4, block=m.Block.TILE, transposed_copy=True)
    out("f4", "fp8 blockwise f32-scale 128x128 + transposed copy (W_gate_up)", [2 * I4, H4], _time_us(
        torch, lambda: m.fp8bw_quantize_f32(w4, block=m.Block.TILE, codes=fw4[0], scales=fw4[1], codes_col=fw4[2],
                                            scales_col=fw4[3], transposed_copy=True), 10),
        nbytes=nw * 2 + 2 * nw + 8 * (nw // 16384))
    fd = m.fp8bw_quantize_f32(dyg4, block=m.Block.DUAL)
    F32S = m.Format.FP8_B128_F32
    out("f4", "fp8 blockwise f32-scale FPROP gate_up", [T4, 2 * I4, H4], _time_us(torch, lambda: m.mx_gemm(
        m.Operand(F32S, f4[0], f4[1]), m.Operand(F32S, fw4[0], fw4[1], block=m.Block.TILE), T4, 2 * I4, H4, out=y4),
        5), flops=f, peak=PEAK_FP8_TFLOPS)
    out("f4", "fp8 blockwise f32-scale DGRAD gate_up (transposed 128x128 copy)", [T4, H4, 2 * I4], _time_us(
        torch, lambda: m.mx_gemm(m.Operand(F32S, fd[0], fd[1]), m.Operand(F32S, fw4[2], fw4[3], block=m.Block.TILE),
                                 T4, H4, 2 * I4, out=dx4), 5), flops=f, peak=PEAK_FP8_TFLOPS)
    out("f4", "fp8 blockwise f32-scale WGRAD gate_up (columnwise copies)", [2 * I4, H4, T4], _time_us(
        torch, lambda: m.mx_gemm(m.Operand(F32S, fd[2], fd[3]), m.Operand(F32S, f4[2], f4[3]), 2 * I4, H4, T4,
                                 out=dw4), 5), flops=f, peak=PEAK_FP8_TFLOPS)
    del x4, w4, wt4, dyg4, dd, d4, y4, dx4, dw4, xo, b4, bw4, f4, fw4, fd
    torch.cuda.empty_cache()

    # ---- Qwen3-30B-A3B-shaped MoE layer, NVFP4 (tokens 8192, hidden 2048, 128 experts, I 768, top-8)
    d = synth.config3()
    T3, H3 = d["x"].shape
    E, N2, _ = d["w_gu"].shape
    I3 = N2 // 2
    lg = d["logits"]
    top = np.argsort(-lg, axis=1, kind="stable")[:, :d["topk"]]          # host routing
    pairs = np.stack([np.repeat(np.arange(T3), d["topk"]), top.reshape(-1)], axis=1)
    order = np.lexsort((pairs[:, 0], pairs[:, 1]))
    row_token = pairs[order, 0].astype(np.int32)
    off = np.zeros(E + 1, dtype=np.int32)
    np.add.at(off, pairs[:, 1] + 1, 1)
    off = np.cumsum(off).astype(np.int32)
    Mr = len(row_token)

    def bf(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)

    x3 = bf(d["x"])
    cx3, sx3, Sx3 = m.nvfp4_quantize(x3)
    wgu = bf(d["w_gu"].reshape(E * N2, H3)).view(E, N2, H3)
    wdn = bf(d["w_dn"].reshape(E * H3, I3)).view(E, H3, I3)
    cgu = torch.empty((E, N2, H3 // 2), dtype=torch.uint8, device=dev)
    sgu = torch.empty((E, N2, H3 // 16), dtype=torch.uint8, device=dev)
    Sgu = torch.empty(E, dtype=torch.float32, device=dev)
    cdn = torch.empty((E, H3, I3 // 2), dtype=torch.uint8, device=dev)
    sdn = torch.empty((E, H3, I3 // 16), dtype=torch.uint8, device=dev)
    Sdn = torch.empty(E, dtype=torch.float32, device=dev)
    for e in range(E):
        m.nvfp4_quantize(wgu[e], gs=m.GScale.PER_TENSOR, codes=cgu[e], block_scales=sgu[e], gscales=Sgu[e:e + 1])
        m.nvfp4_quantize(wdn[e], gs=m.GScale.PER_TENSOR, codes=cdn[e], block_scales=sdn[e], gscales=Sdn[e:e + 1])
    off_d = torch.from_numpy(off).to(dev)
    idx_d = torch.from_numpy(row_token).to(dev)
    A = m.Operand(m.Format.NVFP4, cx3, sx3, Sx3, gs=m.GScale.PER_ROW)
    Bgu = m.Operand(m.Format.NVFP4, cgu.view(E * N2, H3 // 2), sgu, Sgu, gs=m.GScale.PER_TENSOR)
    gu = torch.empty((Mr, N2), dtype=torch.bfloat16, device=dev)
    out("a8", "MoE grouped gate_up (row gather, 128 experts)", [Mr, N2, H3], _time_us(torch, lambda: m.mx_gemm(
        A, Bgu, Mr, N2, H3, out=gu, group_row_offsets=off_d, a_row_index=idx_d, a_rows=T3), 10),
        flops=2.0 * Mr * N2 * H3, peak=PEAK_F16_TFLOPS)
    h = torch.empty((Mr, I3), dtype=torch.bfloat16, device=dev)
    out("a8", "MoE SwiGLU", [Mr, I3], _time_us(torch, lambda: m.mx_swiglu(gu, I3, out=h), 10),
        nbytes=Mr * N2 * 2 + Mr * I3 * 2)
    hf = torch.empty_like(h)
    out("f3", "MoE grouped gate_up with SwiGLU in the epilogue (writes H)", [Mr, N2, H3], _time_us(
        torch, lambda: m.mx_gemm_swiglu(A, Bgu, Mr, I3, H3, out=hf, group_row_offsets=off_d, a_row_index=idx_d,
                                        a_rows=T3), 10), flops=2.0 * Mr * N2 * H3, peak=PEAK_F16_TFLOPS)
    del hf
    ch, sh, Sh = m.nvfp4_quantize(h)
    out("a8", "MoE per-token Q(H)", [Mr, I3], _time_us(torch, lambda: m.nvfp4_quantize(
        h, codes=ch, block_scales=sh, gscales=Sh), 10), nbytes=Mr * I3 * 2 + Mr * I3 // 2 + Mr * I3 // 16 + Mr * 4)
    Bdn = m.Operand(m.Format.NVFP4, cdn.view(E * H3, I3 // 2), sdn, Sdn, gs=m.GScale.PER_TENSOR)
    y3 = torch.empty((Mr, H3), dtype=torch.bfloat16, device=dev)
    out("a8", "MoE grouped down", [Mr, H3, I3], _time_us(torch, lambda: m.mx_gemm(
        m.Operand(m.Format.NVFP4, ch, sh, Sh, gs=m.GScale.PER_ROW), Bdn, Mr, H3, I3, out=y3,
        group_row_offsets=off_d), 10), flops=2.0 * Mr * H3 * I3, peak=PEAK_F16_TFLOPS)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time bound for the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip the device-copy and host-call probes (keeps traced runs to the step)")
    ap.add_argument("--eager", action="store_true",
                    help="time plain launches instead of HIP-graph replays")
    ap.add_argument("--overlap", action="store_true",
                    help="capture the weight path (Q(W), DQ(W)) on a second stream (measured "
                         "slower on MI355X: 83.0 vs 73.7 us per step)")
    ap.add_argument("--rows", action="store_true",
                    help="only time each hot-path row at the other configurations' shapes "
                         "(one JSON line per measurement)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy of known size (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(the quantizers shard by rows with no exchange; see the design notes). "
              f"Asked for --gpus {args.gpus} (WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import microscaling_quantization_block_amd as m
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.rows:
        rows_report()
        return
    m.lib()
    log("generating synthetic inputs (seeded)")
    data = synth.config2()
    sets = make_sets(m, torch, data)
    torch.cuda.synchronize()

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(m, sets[i % SETS])
    torch.cuda.synchronize()

    log(f"timing {args.steps} eager steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(m, sets[i % SETS])
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) / args.steps * 1e3

    # per-stage timing: HIP events around each stage, on the stream the
    # library launches on (torch's current stream).  A spin kernel ahead of
    # each step keeps the GPU busy while the host enqueues the four stages, so
    # the stages run back to back and each event pair brackets its kernels,
    # not the host's launch overhead.
    spin = spin_cycles(torch, SPIN_US)
    log(f"per-stage timing, {args.steps} eager steps, each behind a {SPIN_US:.0f} us spin")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        torch.cuda._sleep(spin)
        step(m, sets[i % SETS], events[i])
    torch.cuda.synchronize()

    ms_graph = None
    if not args.eager:
        log("capturing one HIP graph per buffer set")
        side = torch.cuda.Stream()              # default priority
        graphs = []
        for s_ in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                if args.overlap:
                    step_concurrent(m, s_, side, torch)
                else:
                    step(m, s_)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % SETS].replay()
        torch.cuda.synchronize()
        log(f"timing {args.steps} graph-replayed steps")
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % SETS].replay()
        torch.cuda.synchronize()
        ms_graph = (time.perf_counter() - t0) / args.steps * 1e3
    # the headline is the faster of the two ways of launching the same step
    graph_wins = ms_graph is not None and ms_graph < ms_eager
    ms_step = ms_graph if graph_wins else ms_eager

    names = ["quantize_x_nvfp4_1x16_per_token", "quantize_dequantize_w_nvfp4_16x16_per_tensor",
             "gemm_fprop_nvfp4", "gemm_dgrad_bf16_dequantized"]
    stage_ms = [sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / args.steps for j in range(4)]
    kernels = {}
    for j, nm in enumerate(names):
        us = stage_ms[j] * 1e3
        d = {"us": round(us, 2)}
        if j in (0, 1):
            b = [BYTES_QX, BYTES_QDQW][j]
            gbps = b / (us * 1e-6) / 1e9
            d.update(bytes=b, GBps=round(gbps, 1), frac_hbm=round(gbps / PEAK_HBM_GBPS, 4))
        else:
            f = FLOPS_FPROP if j == 2 else FLOPS_DGRAD
            tf = f / (us * 1e-6) / 1e12
            d.update(flops=f, TFLOPs=round(tf, 1), frac_mfma=round(tf / PEAK_F16_TFLOPS, 4))
            if j == 2:
                d["frac_fp4_peak"] = round(tf / PEAK_FP4_TFLOPS, 4)
        kernels[nm] = d
    # the dominant kernel, timed again over runs of back-to-back launches (an
    # event pair around every launch adds its own packets to each figure)
    dom = max(range(4), key=lambda j: stage_ms[j])
    reps = max(args.steps // 10, 2)
    log(f"roofline kernel {names[dom]}: {reps} runs of {SETS} back-to-back launches")
    dom_us = batch_us(torch, stages(m)[dom], sets, spin_cycles(torch, BATCH_SPIN_US), reps)
    how = (f"HIP events around {reps} runs of {SETS} back-to-back launches (one per buffer set), "
           "each run behind a spin kernel")
    if dom >= 2:
        f = FLOPS_FPROP if dom == 2 else FLOPS_DGRAD
        tf = f / (dom_us * 1e-6) / 1e12
        roofline = dict(kernel=names[dom], bound="mfma", achieved=round(tf, 1), peak=PEAK_F16_TFLOPS,
                        unit="TFLOP/s", frac=round(tf / PEAK_F16_TFLOPS, 4),
                        traffic=measured_traffic(names[dom]), us_per_launch=round(dom_us, 2), timing=how)
    else:
        b = [BYTES_QX, BYTES_QDQW][dom]
        gbps = b / (dom_us * 1e-6) / 1e9
        roofline = dict(kernel=names[dom], bound="hbm", achieved=round(gbps, 1), peak=PEAK_HBM_GBPS,
                        unit="GB/s", frac=round(gbps / PEAK_HBM_GBPS, 4),
                        traffic=measured_traffic(names[dom]), us_per_launch=round(dom_us, 2), timing=how)
    value = (FLOPS_FPROP + FLOPS_DGRAD) / (ms_step * 1e-3) / 1e12
    qbytes = BYTES_QX + BYTES_QDQW
    qus = (stage_ms[0] + stage_ms[1]) * 1e3
    out = {
        "metric": "MX/NVFP4 quantize GB/s + block-scaled GEMM TFLOP/s (% of gfx950 peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_eager": round(ms_eager, 4),
        "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 4),
        "launch": ("hip_graph" + (", weight path (Q(W) with DQ(W)) on a second stream" if args.overlap else "")
                   if graph_wins else "eager (back-to-back launches on one stream)"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 (e2m1/e4m3/fp32) -> f16 MFMA, f32 accumulate; bf16 MFMA for DGRAD",
        "data": "synthetic",
        "config": {"workload": "nvfp4_linear_tokens4096_hidden2048_out768",
                   "stages": "per-token Q(X) 4096x2048, 16x16 Q(W) 768x2048 with DQ(W) in the same pass, "
                             "FPROP 4096x768x2048, dequantized-backward DGRAD 4096x2048x768",
                   "tokens": M, "hidden": K, "out_features": N, "buffer_sets": SETS},
        "quantize_GBps": round(qbytes / (qus * 1e-6) / 1e9, 1),
        "gemm_TFLOPs": round((FLOPS_FPROP + FLOPS_DGRAD) / ((stage_ms[2] + stage_ms[3]) * 1e-3) / 1e12, 1),
        "kernels": kernels,
        "roofline": roofline,
        "measured_reference": None if args.no_reference else measured_reference(m, torch),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(data, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
