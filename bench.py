#!/usr/bin/env python3
"""Benchmark of the microscaling hot path on one MI355X.

Headline workload: the Llama-3-8B-shaped dense MLP in NVFP4 of the NVFP4
pretraining pages (sequence 8192 x micro-batch 4 = 32768 tokens, hidden 4096,
intermediate 14336).  One step = one training pass over one batch of both
linears, gate_up (4096 -> 28672) and down (14336 -> 4096), each:
   1. Q(X)  rowwise 1x16, per-token S, RNE            (FPROP operand), then
            columnwise 16x1, per-tensor S, RNE        (WGRAD operand); the
            rowwise pass also accumulates the tensor amax
   2. (the columnwise copy of step 1)
   3. Q(W)  16x16 tiles, per-tensor S, RNE, with the transposed copy (the 16x16
            copy of W^T, written in the same pass)        (FPROP; DGRAD)
   4. FPROP  Y  = Q(X) Q(W)^T                         (BF16 out)
   5. Q(dY) rowwise 1x16, per-token S, stochastic rounding (seed 0, stream 0), then
            columnwise 16x1, per-tensor S, stochastic rounding (stream 1)
   6. (the columnwise copy of step 5)
   7. DGRAD dX = Q(dY) Q(W)                           (the transposed 16x16 copy)
   8. WGRAD dW = Q(dY)^T Q(X)                         (the two columnwise copies)
Each linear is measured on its own seeded inputs (the SwiGLU between them is
not part of this path).  Inputs are seeded synthetic tensors (synth.mlp_tensor;
the pages' model and dataset stand in as shapes and distributions only),
resident in HBM before timing; a step moves about 9 GB, far more than the
256 MB last-level cache.

Prints ONE JSON line on stdout.  `value` = the step's GEMM throughput: the six
GEMMs' algorithmic flops (2 M N K each, 34.6 TFLOP per step) over the whole
step's wall time, quantization included.  Every stage carries a HIP event
pair on the launch stream inside the timed steps; "kernels" gives each
stage's time, GB/s or TFLOP/s and fraction of peak, and "roofline" the stage
with the largest share (its average launch duration from those events).  The
CPU oracle, timed on a bounded sample of the same step, is "cpu_baseline".
"config2" repeats the smaller NVFP4 linear of the second configuration
(4096 tokens, 2048 -> 768, with the dequantized-backward DGRAD).
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

T, HID, INTER = 32768, 4096, 14336
PEAK_HBM_GBPS = 8000.0
PEAK_F16_TFLOPS = 2500.0     # dense FP16/BF16 MFMA (the dtype the NVFP4 GEMM issues)
PEAK_FP4_TFLOPS = 10100.0    # dense FP4 MFMA (context for the NVFP4 GEMM)
PEAK_FP8_TFLOPS = 5000.0

# (linear, input, weight, output gradient, K, N)
LINEARS = [("gate_up", "x", "w_gu", "dy_gu", HID, 2 * INTER), ("down", "h", "w_dn", "dy_dn", INTER, HID)]
STEP_FLOPS = sum(3 * 2 * T * N * K for _, _, _, _, K, N in LINEARS)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


COPY_BYTES = 256 << 20
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "microscaling_quantization_block_amd", "csrc", "gemm.hip")


def measured_reference(m, torch):
    """Context for the spec peaks: the bandwidth of a plain device copy of
    COPY_BYTES (read + write bytes over time, HIP events, 20 copies) and of a
    reduction that only reads them, and the
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
    del dst
    # read-only: torch's sum over the same bytes as float32 (a reduction reads
    # everything once and writes a scalar)
    f = src.view(torch.float32)
    for _ in range(3):
        f.sum()
    torch.cuda.synchronize()
    a.record()
    for _ in range(20):
        f.sum()
    b.record()
    torch.cuda.synchronize()
    read_gbps = COPY_BYTES * 20 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, f
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
            "read_GBps": round(read_gbps, 1), "read_frac_of_hbm_peak": round(read_gbps / PEAK_HBM_GBPS, 4),
            "host_us_per_call": round(host_us, 2),
            "note": "device copy of 256 MiB (read + write bytes); a float32 sum over the same 256 MiB (read "
                    "bytes); host time of one Python -> C ABI call"}


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


# ---------------------------------------------------------------- the step

def make_buffers(m, torch):
    """Inputs (seeded, on the device) and every output of the step."""
    import synth
    dev = "cuda"
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
    bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)
    b = {}
    for lin, xn, wn, dn, K, N in LINEARS:
        d = dict(x=synth.mlp_tensor(5, xn, dev), w=synth.mlp_tensor(5, wn, dev), dy=synth.mlp_tensor(5, dn, dev),
                 K=K, N=N)
        d.update(cx=u8(T, K // 2), sx=u8(T, K // 16), Sx=f32(T),
                 cxc=u8(K, T // 2), sxc=u8(K, T // 16), Sxc=f32(1),
                 cw=u8(N, K // 2), sw=u8(N // 16, K // 16), Sw=f32(1),
                 cwt=u8(K, N // 2), swt=u8(K // 16, N // 16),
                 cd=u8(T, N // 2), sd=u8(T, N // 16), Sd=f32(T),
                 cdc=u8(N, T // 2), sdc=u8(N, T // 16), Sdc=f32(1),
                 y=bf(T, N), dx=bf(T, K), dw=bf(N, K))
        b[lin] = d
    return b


def stages(m, b):
    """The step's 12 stages: (name, fn, algorithmic bytes or None, flops or None)."""
    out = []
    NV = m.Format.NVFP4
    for lin, _, _, _, K, N in LINEARS:
        d = b[lin]

        def qx(d=d):
            # rowwise per-token copy, then the columnwise per-tensor copy (its
            # tensor amax accumulated by the rowwise pass)
            m.nvfp4_quantize_rowcol(d["x"], codes=d["cx"], block_scales=d["sx"], gscales=d["Sx"],
                                    codes_col=d["cxc"], block_scales_col=d["sxc"], gscale_col=d["Sxc"])

        def qw(d=d):
            # the 16x16 copy and its transposed copy (DGRAD's B) from one pass
            m.nvfp4_quantize_tile_t(d["w"], gs=m.GScale.PER_TENSOR, codes=d["cw"], block_scales=d["sw"],
                                    codes_t=d["cwt"], block_scales_t=d["swt"], gscales=d["Sw"])

        def fprop(d=d, K=K, N=N):
            m.mx_gemm(m.Operand(NV, d["cx"], d["sx"], d["Sx"], gs=m.GScale.PER_ROW),
                      m.Operand(NV, d["cw"], d["sw"], d["Sw"], block=m.Block.TILE, gs=m.GScale.PER_TENSOR),
                      T, N, K, out=d["y"])

        def qd(d=d):
            m.nvfp4_quantize_rowcol(d["dy"], rnd=m.Round.SR, seed=0, codes=d["cd"], block_scales=d["sd"],
                                    gscales=d["Sd"], codes_col=d["cdc"], block_scales_col=d["sdc"],
                                    gscale_col=d["Sdc"])

        def dgrad(d=d, K=K, N=N):
            m.mx_gemm(m.Operand(NV, d["cd"], d["sd"], d["Sd"], gs=m.GScale.PER_ROW),
                      m.Operand(NV, d["cwt"], d["swt"], d["Sw"], block=m.Block.TILE, gs=m.GScale.PER_TENSOR),
                      T, K, N, out=d["dx"])

        def wgrad(d=d, K=K, N=N):
            m.mx_gemm(m.Operand(NV, d["cdc"], d["sdc"], d["Sdc"], gs=m.GScale.PER_TENSOR),
                      m.Operand(NV, d["cxc"], d["sxc"], d["Sxc"], gs=m.GScale.PER_TENSOR), N, K, T, out=d["dw"])

        nx, nw, nd = T * K, N * K, T * N
        f = 2 * T * N * K
        # the two copies of x (and of dY) read it twice: the rowwise pass, which
        # also accumulates the tensor amax, and the columnwise pass
        rc = lambda n, rows: 2 * n * 2 + 2 * (n // 2 + n // 16) + rows * 4 + 4
        out += [(f"{lin}_quantize_x_rowwise_and_colwise_rne", qx, rc(nx, T), None),
                # ... and the weight (two reads) with its transposed copy
                (f"{lin}_quantize_w_16x16_per_tensor_rne", qw, 2 * nw * 2 + 2 * (nw // 2 + nw // 256) + 4, None),
                (f"{lin}_gemm_fprop_nvfp4", fprop, None, f),
                (f"{lin}_quantize_dy_rowwise_and_colwise_sr", qd, rc(nd, T), None),
                (f"{lin}_gemm_dgrad_nvfp4", dgrad, None, f),
                (f"{lin}_gemm_wgrad_nvfp4", wgrad, None, f)]
    return out


def stage_entry(us, nbytes, flops):
    d = {"us": round(us, 1)}
    if nbytes is not None:
        gbps = nbytes / (us * 1e-6) / 1e9
        d.update(bytes=int(nbytes), GBps=round(gbps, 1), frac_hbm=round(gbps / PEAK_HBM_GBPS, 4))
    else:
        tf = flops / (us * 1e-6) / 1e12
        d.update(flops=int(flops), TFLOPs=round(tf, 1), frac_mfma=round(tf / PEAK_F16_TFLOPS, 4),
                 frac_fp4_peak=round(tf / PEAK_FP4_TFLOPS, 4))
    return d


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(min_seconds, tokens=256, feats=512):
    """The oracle, as it stands, on a bounded sample of the same step: both
    linears restricted to their first `tokens` tokens and first `feats`
    output features (all K), every stage as the GPU runs it (per-token RNE
    and columnwise copies of X, 16x16 W, SR rowwise and columnwise dY, FPROP,
    DGRAD and WGRAD as float64 dequantize-then-matmul), repeated until
    `min_seconds` have passed.  Inputs are synth.mlp_tensor's tensors (the
    GPU's inputs) copied to the host before the sample is cut."""
    import numpy as np
    import torch
    import synth
    from oracle import formats as F, nvfp4 as ON, gemm as G
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = len(os.sched_getaffinity(0))
    host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    sample = []
    for lin, xn, wn, dn, K, N in LINEARS:
        x = synth.mlp_tensor(5, xn, "cuda")[:tokens]
        w = synth.mlp_tensor(5, wn, "cuda")[:feats]
        dy = synth.mlp_tensor(5, dn, "cuda")[:tokens, :feats]
        sample.append((F.bf16_bits_to_f64(host(x)), F.bf16_bits_to_f64(host(w)), F.bf16_bits_to_f64(host(dy))))
        del x, w, dy
    torch.cuda.empty_cache()
    flops = sum(3 * 2 * tokens * feats * K for _, _, _, _, K, _ in LINEARS)
    reps = 0
    t0 = time.perf_counter()
    while True:
        for xv, wv, dyv in sample:
            xc, xs, xS = ON.quantize_rowwise(xv, "per_row")
            xcc, xcs, xcS = ON.quantize_colwise(xv)
            wc, ws, wS = ON.quantize_tile16(wv)
            dc, ds, dS = ON.quantize_rowwise(dyv, "per_row", rnd="sr", seed=0, stream_id=0)
            dcc, dcs, dcS = ON.quantize_colwise(dyv, rnd="sr", seed=0, stream_id=1)
            x64 = ON.dequantize_f64(xc, xs, xS, "1x16", "per_row")
            w64 = ON.dequantize_f64(wc, ws, wS, "16x16", "per_tensor")
            d64 = ON.dequantize_f64(dc, ds, dS, "1x16", "per_row")
            y = F.bf16_rne(G.gemm_f64(x64, w64))
            dx = F.bf16_rne(G.gemm_f64(d64, w64.T.copy()))
            dw = F.bf16_rne(G.gemm_f64(ON.dequantize_f64(dcc, dcs, dcS, "1x16", "per_tensor"),
                                       ON.dequantize_f64(xcc, xcs, xcS, "1x16", "per_tensor")))
            assert y.shape == (tokens, feats) and dx.shape == xv.shape and dw.shape == wv.shape
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    t_step = el / reps
    return dict(value=flops / t_step / 1e12, unit="TFLOP/s", cores=int(blas_threads), kind="oracle",
                sample=(f"the step restricted to the first {tokens} tokens and {feats} output features of "
                        f"each linear (all 16 stages, GEMMs as float64 dequantize-then-matmul), repeated "
                        f"{reps} times in {el:.1f} s; quantizers single-threaded NumPy, matmuls on "
                        f"{blas_threads} BLAS threads"),
                seconds_per_sample_step=round(t_step, 3), sample_gemm_flops=int(flops))


def oracle_rates(min_seconds=1.0):
    """The oracle's own throughput per configuration on this host (part of the
    CPU-baseline leg; no GPU): each operation on the named sample, repeated for
    at least `min_seconds`; one JSON line each.  Quantizers are single-threaded
    NumPy, matmuls run on the BLAS threads.  The config-4/5 samples are rows of
    tensors drawn with NumPy at the same shapes and distributions as the GPU's
    device-generated ones."""
    import numpy as np
    import synth
    from oracle import formats as F, nvfp4 as ON, mxfp8 as OM, gemm as G
    cores = len(os.sched_getaffinity(0))

    def timed(fn):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= min_seconds:
                return el / n

    def rec(cfg, what, sample, fn, elems=None, nbytes=None, flops=None):
        sec = timed(fn)
        d = dict(cfg=cfg, what=what, sample=sample, seconds=round(sec, 4), cores=cores)
        if elems:
            d["Melem_s"] = round(elems / sec / 1e6, 2)
        if nbytes:
            d["GBps"] = round(nbytes / sec / 1e9, 3)
        if flops:
            d["GFLOPs"] = round(flops / sec / 1e9, 2)
        print(json.dumps(d), flush=True)

    f64 = F.bf16_bits_to_f64
    d = synth.config1()
    x, w = f64(d["x"]), f64(d["w"])
    n = x.size
    rec(1, "mxfp8 1x32 quantize", "whole 256x512", lambda: OM.quantize_rowwise(x), n, 3 * n + n // 32)
    c, sc = OM.quantize_rowwise(x)
    cw, sw = OM.quantize_rowwise(w)
    rec(1, "mxfp8 dequantize", "whole", lambda: OM.dequantize_bf16(c, sc), n, n + n // 32 + 2 * n)
    rec(1, "mxfp8 GEMM f64 (dequantize, then matmul)", "whole 256x512x256",
        lambda: G.gemm_f64(OM.dequantize_f64(c, sc), OM.dequantize_f64(cw, sw)), flops=2 * 256 * 256 * 512)
    d = synth.config2()
    x, w, dy = f64(d["x"]), f64(d["w"]), f64(d["dy"])
    n, nw = x.size, w.size
    rec(2, "nvfp4 per-token quantize", "whole 4096x2048", lambda: ON.quantize_rowwise(x, "per_row"), n,
        2 * n + n // 2 + n // 16 + 4096 * 4)
    rec(2, "nvfp4 16x16 weight quantize", "whole 768x2048", lambda: ON.quantize_tile16(w), nw,
        4 * nw + nw // 2 + nw // 256 + 4)
    xc, xs, xS = ON.quantize_rowwise(x, "per_row")
    wc, wsb, wS = ON.quantize_tile16(w)
    rec(2, "nvfp4 FPROP f64", "whole 4096x768x2048",
        lambda: G.gemm_f64(ON.dequantize_f64(xc, xs, xS, "1x16", "per_row"),
                           ON.dequantize_f64(wc, wsb, wS, "16x16", "per_tensor")), flops=2 * 4096 * 768 * 2048)
    rec(2, "nvfp4 dequantize (W)", "whole", lambda: ON.dequantize_bf16(wc, wsb, wS, "16x16", "per_tensor"), nw,
        nw // 2 + nw // 256 + 2 * nw)
    wdq = f64(ON.dequantize_bf16(wc, wsb, wS, "16x16", "per_tensor"))
    rec(2, "dequantized-backward DGRAD f64", "whole 4096x2048x768", lambda: G.gemm_f64(dy, wdq.T.copy()),
        flops=2 * 4096 * 2048 * 768)
    d = synth.config3()
    x3 = f64(d["x"][:2048])
    n = x3.size
    rec(3, "nvfp4 per-token quantize (X)", "2048 of 8192 tokens", lambda: ON.quantize_rowwise(x3, "per_row"), n,
        2 * n + n // 2 + n // 16 + 2048 * 4)
    we = f64(d["w_gu"][0])
    rec(3, "nvfp4 expert weight quantize (one S over gate and up)", "1 of 128 experts",
        lambda: ON.quantize_rowwise(we, "per_tensor"), we.size, 4 * we.size + we.size // 2 + we.size // 16 + 4)
    wc, ws, wS = ON.quantize_rowwise(we, "per_tensor")
    xc, xs, xS = ON.quantize_rowwise(x3[:512], "per_row")
    rec(3, "grouped gate_up GEMM f64, one expert", "512 rows x 1536 x 2048",
        lambda: G.gemm_f64(ON.dequantize_f64(xc, xs, xS, "1x16", "per_row"),
                           ON.dequantize_f64(wc, ws, wS, "1x16", "per_tensor")), flops=2 * 512 * 1536 * 2048)
    for cfg in (4, 5):
        K = 4096
        xs_ = f64(synth.normal_bf16((256, K), 1.0, cfg, 0))
        ws_ = f64(synth.normal_bf16((1024, K), 0.02, cfg, 1))
        n = xs_.size
        if cfg == 4:
            rec(4, "mxfp8 dual (rowwise + columnwise) quantize", "256 x 4096",
                lambda: (OM.quantize_rowwise(xs_), OM.quantize_colwise(xs_)), n, 4 * n + 2 * (n // 32))
            rec(4, "mxfp8 32x32 weight quantize", "1024 x 4096", lambda: OM.quantize_tile32(ws_), ws_.size,
                3 * ws_.size)
            a, sa = OM.quantize_rowwise(xs_)
            b, sb = OM.quantize_tile32(ws_)
            rec(4, "mxfp8 FPROP f64", "256 x 1024 x 4096 of 8192 x 24576 x 4096",
                lambda: G.gemm_f64(OM.dequantize_f64(a, sa), OM.dequantize_f64(b, sb, "32x32")),
                flops=2 * 256 * 1024 * K)
        else:
            rec(5, "nvfp4 per-token RNE quantize", "256 x 4096", lambda: ON.quantize_rowwise(xs_, "per_row"), n,
                2 * n + n // 2 + n // 16 + 256 * 4)
            rec(5, "nvfp4 per-token SR quantize", "256 x 4096",
                lambda: ON.quantize_rowwise(xs_, "per_row", rnd="sr"), n, 2 * n + n // 2 + n // 16 + 256 * 4)
            rec(5, "nvfp4 columnwise SR quantize", "256 x 4096", lambda: ON.quantize_colwise(xs_, rnd="sr"), n,
                4 * n + n // 2 + n // 16 + 4)
            rec(5, "nvfp4 16x16 weight quantize", "1024 x 4096", lambda: ON.quantize_tile16(ws_), ws_.size,
                4 * ws_.size + ws_.size // 2 + ws_.size // 256 + 4)
            a, sa, Sa = ON.quantize_rowwise(xs_, "per_row")
            b, sb, Sb = ON.quantize_tile16(ws_)
            rec(5, "nvfp4 FPROP f64", "256 x 1024 x 4096 of 32768 x 28672 x 4096",
                lambda: G.gemm_f64(ON.dequantize_f64(a, sa, Sa, "1x16", "per_row"),
                                   ON.dequantize_f64(b, sb, Sb, "16x16", "per_tensor")), flops=2 * 256 * 1024 * K)


# ---------------------------------------------------------------- config 2

def config2_step(m, torch, steps):
    """The second configuration's NVFP4 linear (4096 tokens, 2048 -> 768):
    per-token Q(X), 16x16 Q(W) with DQ(W) in the same pass, FPROP and the
    dequantized-backward BF16 DGRAD, over ten rotating buffer sets (> 512 MB)."""
    import numpy as np
    import synth
    M, K, N = 4096, 2048, 768
    data = synth.config2()
    dev = "cuda"

    def bfd(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    x0, w0, dy0 = bfd(data["x"]), bfd(data["w"]), bfd(data["dy"])
    sets = []
    for _ in range(10):
        s = dict(x=x0.clone(), w=w0.clone(), dy=dy0.clone())
        s.update(cx=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                 sx=torch.empty((M, K // 16), dtype=torch.uint8, device=dev),
                 Sx=torch.empty(M, dtype=torch.float32, device=dev),
                 cw=torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
                 sw=torch.empty((N // 16, K // 16), dtype=torch.uint8, device=dev),
                 Sw=torch.empty(1, dtype=torch.float32, device=dev),
                 y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                 wdq=torch.empty((N, K), dtype=torch.bfloat16, device=dev),
                 dx=torch.empty((M, K), dtype=torch.bfloat16, device=dev))
        sets.append(s)

    def step(s):
        m.nvfp4_quantize(s["x"], gs=m.GScale.PER_ROW, codes=s["cx"], block_scales=s["sx"], gscales=s["Sx"])
        m.nvfp4_quantize_dq(s["w"], codes=s["cw"], block_scales=s["sw"], gscales=s["Sw"], dq=s["wdq"])
        m.mx_gemm(m.Operand(m.Format.NVFP4, s["cx"], s["sx"], s["Sx"], gs=m.GScale.PER_ROW),
                  m.Operand(m.Format.NVFP4, s["cw"], s["sw"], s["Sw"], block=m.Block.TILE,
                            gs=m.GScale.PER_TENSOR), M, N, K, out=s["y"])
        m.mx_gemm(m.Operand(m.Format.BF16, s["dy"], block=m.Block.NONE),
                  m.Operand(m.Format.BF16, s["wdq"], block=m.Block.NONE, transposed=True), M, K, N,
                  out=s["dx"])

    for i in range(20):
        step(sets[i % 10])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(sets[i % 10])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    flops = 2 * (2 * M * N * K)
    return {"workload": "nvfp4_linear_tokens4096_hidden2048_out768 (Q(X), Q(W)+DQ(W), FPROP, "
                        "dequantized-backward DGRAD)",
            "ms_per_step": round(ms, 4), "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1), "steps": steps,
            "launch": "eager, ten rotating buffer sets"}


# ---------------------------------------------------------------- --rows

def _time_rot(torch, fns, iters, warm_ms=30.0):
    """Mean time of one launch, cycling over `fns` (one closure per buffer set,
    so that reads come from HBM rather than the last-level cache): warm up for
    about warm_ms (at least one pass over the sets), then HIP events around
    `iters` launches."""
    t0, n = time.perf_counter(), 0
    while n < max(3, len(fns)) or (time.perf_counter() - t0) * 1e3 < warm_ms:
        fns[n % len(fns)]()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(iters):
        fns[i % len(fns)]()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters * 1e3


ROT_BYTES = 640 << 20     # buffer sets per row: enough copies of the inputs to exceed this


def _copies(nbytes):
    return max(2, -(-ROT_BYTES // max(int(nbytes), 1)))


def rows_report():
    """Each hot-path row at the other configurations' shapes: quantizers and
    dequantizers against HBM bandwidth, GEMMs against their dtype's MFMA
    peak, the MoE stages of the Qwen3-30B-A3B-shaped layer.  One JSON line
    per measurement.  Every row cycles over copies of its inputs totalling
    more than 640 MB, so that they come from HBM, not the 256 MB cache."""
    import numpy as np
    import torch
    import microscaling_quantization_block_amd as m
    import synth
    dev = "cuda"

    def out(row, what, shape, us, nbytes=None, flops=None, peak=None, fp4=False, sets=None):
        d = dict(row=row, what=what, shape=shape, us=round(us, 2), buffer_sets=sets)
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

    def quant_row(row, what, x, call, nbytes, iters=10):
        """call(x_copy) -> closure; x copies rotated."""
        n = _copies(x.numel() * 2)
        xs = [x] + [x.clone() for _ in range(n - 1)]
        fns = [call(xi) for xi in xs]
        out(row, what, list(x.shape), _time_rot(torch, fns, iters), nbytes=nbytes, sets=n)
        del xs, fns

    def bfd(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- the small MXFP8 case: 256x512 activations, 256x512x256 GEMM
    d1 = synth.config1()
    x1, w1 = bfd(d1["x"]), bfd(d1["w"])
    n1 = x1.numel()
    c1, s1 = m.mx_quantize(x1)
    quant_row("a1-a3", "mxfp8 1x32 (X, 256x512)", x1, lambda xi: lambda: m.mx_quantize(xi, codes=c1, scales=s1),
              n1 * 2 + n1 + n1 // 32)
    o1 = torch.empty_like(x1)
    out("a4", "mxfp8 dequantize 1x32 -> bf16 (X, 256x512)", [256, 512], _time_rot(torch, [
        (lambda: m.mx_dequantize(m.Format.MXFP8, c1, s1, 256, 512, out=o1))], 50),
        nbytes=n1 + n1 // 32 + n1 * 2, sets=1)
    cw1, sw1 = m.mx_quantize(w1)
    y1 = torch.empty((256, 256), dtype=torch.bfloat16, device=dev)
    out("a5", "mxfp8 GEMM 256x256x512", [256, 256, 512], _time_rot(torch, [
        (lambda: m.mx_gemm(m.Operand(m.Format.MXFP8, c1, s1), m.Operand(m.Format.MXFP8, cw1, sw1),
                           256, 256, 512, out=y1))], 50),
        flops=2.0 * 256 * 256 * 512, peak=PEAK_FP8_TFLOPS, sets=1)

    # ---- the NVFP4 linear: 4096 tokens, 2048 -> 768
    d2 = synth.config2()
    x2, w2, dy2 = bfd(d2["x"]), bfd(d2["w"]), bfd(d2["dy"])
    M2, K2, N2 = 4096, 2048, 768
    n2, nw2 = x2.numel(), w2.numel()
    c2, s2, S2 = m.nvfp4_quantize(x2)
    quant_row("a1-a3", "nvfp4 1x16 per-token RNE (X, 4096x2048)", x2, lambda xi: lambda: m.nvfp4_quantize(
        xi, codes=c2, block_scales=s2, gscales=S2), n2 * 2 + n2 // 2 + n2 // 16 + M2 * 4)
    cw2, sw2, Sw2 = m.nvfp4_quantize(w2, block=m.Block.TILE, gs=m.GScale.PER_TENSOR)
    wdq2 = torch.empty_like(w2)
    quant_row("a1-a4", "nvfp4 16x16 per-tensor + DQ(W) in the same pass (W, 768x2048)", w2, lambda xi: lambda:
              m.nvfp4_quantize_dq(xi, codes=cw2, block_scales=sw2, gscales=Sw2, dq=wdq2),
              2 * nw2 * 2 + nw2 // 2 + nw2 // 256 + 4 + nw2 * 2)
    y2 = torch.empty((M2, N2), dtype=torch.bfloat16, device=dev)
    nsets = _copies(c2.numel() + cw2.numel())
    ops = [(c2.clone(), cw2.clone()) for _ in range(nsets)]
    out("a6", "nvfp4 FPROP 4096x768x2048", [M2, N2, K2], _time_rot(torch, [
        (lambda a=a, b=b: m.mx_gemm(m.Operand(m.Format.NVFP4, a, s2, S2, gs=m.GScale.PER_ROW),
                                    m.Operand(m.Format.NVFP4, b, sw2, Sw2, block=m.Block.TILE,
                                              gs=m.GScale.PER_TENSOR), M2, N2, K2, out=y2)) for a, b in ops], 50),
        flops=2.0 * M2 * N2 * K2, peak=PEAK_F16_TFLOPS, fp4=True, sets=nsets)
    dx2 = torch.empty((M2, K2), dtype=torch.bfloat16, device=dev)
    nsets = _copies(dy2.numel() * 2 + wdq2.numel() * 2)
    ops = [(dy2.clone(), wdq2.clone()) for _ in range(nsets)]
    out("a7", "dequantized-backward DGRAD (BF16) 4096x2048x768", [M2, K2, N2], _time_rot(torch, [
        (lambda a=a, b=b: m.mx_gemm(m.Operand(m.Format.BF16, a, block=m.Block.NONE),
                                    m.Operand(m.Format.BF16, b, block=m.Block.NONE, transposed=True),
                                    M2, K2, N2, out=dx2)) for a, b in ops], 50),
        flops=2.0 * M2 * N2 * K2, peak=PEAK_F16_TFLOPS, sets=nsets)
    del x2, w2, dy2, ops

    # ---- Llama-3-8B-shaped dense MLP, NVFP4 (tokens 32768, hidden 4096, I 14336)
    T5, H5, I5 = 32768, 4096, 14336
    x5 = synth.mlp_tensor(5, "x", dev)
    n = T5 * H5
    cx, sx, Sx = m.nvfp4_quantize(x5)
    quant_row("a1-a3", "nvfp4 1x16 per-token RNE (X)", x5, lambda xi: lambda: m.nvfp4_quantize(
        xi, codes=cx, block_scales=sx, gscales=Sx), n * 2 + n // 2 + n // 16 + T5 * 4)
    quant_row("f2", "nvfp4 1x16 per-token RNE + Four-Over-Six (X)", x5, lambda xi: lambda: m.nvfp4_quantize(
        xi, rnd=m.Round.RNE_4OVER6, codes=cx, block_scales=sx, gscales=Sx), n * 2 + n // 2 + n // 16 + T5 * 4)
    dy5 = synth.mlp_tensor(5, "dy_dn", dev)                  # down-projection output gradient [T, 4096]
    cg, sg, Sg = m.nvfp4_quantize(dy5, rnd=m.Round.SR)
    quant_row("a1-a3", "nvfp4 1x16 per-token SR (dY)", dy5, lambda xi: lambda: m.nvfp4_quantize(
        xi, rnd=m.Round.SR, codes=cg, block_scales=sg, gscales=Sg), n * 2 + n // 2 + n // 16 + T5 * 4)
    cgc, sgc, Sgc = m.nvfp4_quantize(dy5, block=m.Block.COL, gs=m.GScale.PER_TENSOR, rnd=m.Round.SR, stream_id=1)
    quant_row("a1-a3", "nvfp4 16x1 columnwise per-tensor SR (dY^T, WGRAD)", dy5, lambda xi: lambda: m.nvfp4_quantize(
        xi, block=m.Block.COL, gs=m.GScale.PER_TENSOR, rnd=m.Round.SR, stream_id=1, codes=cgc,
        block_scales=sgc, gscales=Sgc), 2 * n * 2 + n // 2 + n // 16 + 4)
    quant_row("f1", "nvfp4 16x1 columnwise + RHT per-tensor SR (dY^T, WGRAD)", dy5, lambda xi: lambda:
              m.nvfp4_quantize_rht(xi, 0x6B2D, rnd=m.Round.SR, codes=cgc, block_scales=sgc, gscales=Sgc),
              2 * n * 2 + n // 2 + n // 16 + 4)
    quant_row("f1", "nvfp4 16x1 columnwise + RHT per-tensor RNE (X^T, WGRAD)", x5, lambda xi: lambda:
              m.nvfp4_quantize_rht(xi, 0x6B2D, codes=cgc, block_scales=sgc, gscales=Sgc),
              2 * n * 2 + n // 2 + n // 16 + 4)
    quant_row("a1-a3", "nvfp4 16x1 columnwise per-tensor RNE (X^T, WGRAD)", x5, lambda xi: lambda: m.nvfp4_quantize(
        xi, block=m.Block.COL, gs=m.GScale.PER_TENSOR, codes=cgc, block_scales=sgc, gscales=Sgc),
        2 * n * 2 + n // 2 + n // 16 + 4)
    rcb = 2 * n * 2 + 2 * (n // 2 + n // 16) + T5 * 4 + 4
    quant_row("a1-a3", "nvfp4 rowwise per-token + columnwise per-tensor, two passes, RNE (X)", x5, lambda xi: lambda:
              m.nvfp4_quantize_rowcol(xi, codes=cx, block_scales=sx, gscales=Sx, codes_col=cgc,
                                      block_scales_col=sgc, gscale_col=Sgc), rcb)
    quant_row("a1-a3", "nvfp4 rowwise per-token + columnwise per-tensor, two passes, SR (dY)", dy5, lambda xi: lambda:
              m.nvfp4_quantize_rowcol(xi, rnd=m.Round.SR, codes=cg, block_scales=sg, gscales=Sg, codes_col=cgc,
                                      block_scales_col=sgc, gscale_col=Sgc), rcb)
    h5 = synth.mlp_tensor(5, "h", dev)
    nh = h5.numel()
    ch5, sh5, Sh5 = m.nvfp4_quantize(h5)
    quant_row("a1-a3", "nvfp4 1x16 per-token RNE, rows of 14336 (H)", h5, lambda xi: lambda: m.nvfp4_quantize(
        xi, codes=ch5, block_scales=sh5, gscales=Sh5), nh * 2 + nh // 2 + nh // 16 + T5 * 4)
    del h5, ch5, sh5
    w5 = synth.mlp_tensor(5, "w_gu", dev)                    # gate_up weight [N, K]
    nw = w5.numel()
    cw, sw, Sw = m.nvfp4_quantize(w5, block=m.Block.TILE, gs=m.GScale.PER_TENSOR)
    quant_row("a1-a3", "nvfp4 16x16 per-tensor (W_gate_up)", w5, lambda xi: lambda: m.nvfp4_quantize(
        xi, block=m.Block.TILE, gs=m.GScale.PER_TENSOR, codes=cw, block_scales=sw, gscales=Sw),
        2 * nw * 2 + nw // 2 + nw // 256 + 4)
    cwt, swt = torch.empty((H5, I5), dtype=torch.uint8, device=dev), torch.empty((H5 // 16, 2 * I5 // 16), dtype=torch.uint8, device=dev)
    quant_row("a1-a3", "nvfp4 16x16 per-tensor + transposed copy (W_gate_up)", w5, lambda xi: lambda:
              m.nvfp4_quantize_tile_t(xi, codes=cw, block_scales=sw, codes_t=cwt, block_scales_t=swt, gscales=Sw),
              2 * nw * 2 + 2 * (nw // 2 + nw // 256) + 4)
    del cwt, swt
    quant_row("f2", "nvfp4 16x16 per-tensor + Four-Over-Six (W_gate_up)", w5, lambda xi: lambda: m.nvfp4_quantize(
        xi, block=m.Block.TILE, gs=m.GScale.PER_TENSOR, rnd=m.Round.RNE_4OVER6, codes=cw, block_scales=sw,
        gscales=Sw), 2 * nw * 2 + nw // 2 + nw // 256 + 4)
    nsets = _copies(nw // 2)
    cws = [cw] + [cw.clone() for _ in range(nsets - 1)]
    wdq = torch.empty_like(w5)
    out("a4", "nvfp4 dequantize 16x16 -> bf16 (W_gate_up)", [2 * I5, H5], _time_rot(torch, [
        (lambda c=c: m.mx_dequantize(m.Format.NVFP4, c, sw, 2 * I5, H5, block=m.Block.TILE, gscales=Sw,
                                     gs=m.GScale.PER_TENSOR, out=wdq)) for c in cws], 10),
        nbytes=nw // 2 + nw // 256 + 4 + nw * 2, sets=nsets)
    del cws, wdq, w5
    # GEMMs of the gate_up linear: operands rotated over copies of the codes
    f = 2.0 * T5 * 2 * I5 * H5
    y5 = torch.empty((T5, 2 * I5), dtype=torch.bfloat16, device=dev)
    nsets = _copies(cx.numel() + cw.numel())
    ops = [(cx.clone(), cw.clone()) for _ in range(nsets)]
    out("a6", "nvfp4 FPROP gate_up", [T5, 2 * I5, H5], _time_rot(torch, [
        (lambda a=a, b=b: m.mx_gemm(m.Operand(m.Format.NVFP4, a, sx, Sx, gs=m.GScale.PER_ROW),
                                    m.Operand(m.Format.NVFP4, b, sw, Sw, block=m.Block.TILE, gs=m.GScale.PER_TENSOR),
                                    T5, 2 * I5, H5, out=y5)) for a, b in ops], 4),
        flops=f, peak=PEAK_F16_TFLOPS, fp4=True, sets=nsets)
    del y5, ops
    dyg = synth.mlp_tensor(5, "dy_gu", dev)                  # gate_up output gradient
    cdg, sdg, Sdg = m.nvfp4_quantize(dyg, rnd=m.Round.SR)
    dx5 = torch.empty((T5, H5), dtype=torch.bfloat16, device=dev)
    nsets = _copies(cdg.numel() + cw.numel())
    ops = [(cdg.clone(), cw.clone()) for _ in range(nsets)]
    out("a6", "nvfp4 DGRAD gate_up (16x16 weight read transposed)", [T5, H5, 2 * I5], _time_rot(torch, [
        (lambda a=a, b=b: m.mx_gemm(m.Operand(m.Format.NVFP4, a, sdg, Sdg, gs=m.GScale.PER_ROW),
                                    m.Operand(m.Format.NVFP4, b, sw, Sw, block=m.Block.TILE, gs=m.GScale.PER_TENSOR,
                                              transposed=True), T5, H5, 2 * I5, out=dx5)) for a, b in ops], 4),
        flops=f, peak=PEAK_F16_TFLOPS, fp4=True, sets=nsets)
    del ops
    cwt, swt = torch.empty((H5, I5), dtype=torch.uint8, device=dev), torch.empty((H5 // 16, 2 * I5 // 16), dtype=torch.uint8, device=dev)
    w5 = synth.mlp_tensor(5, "w_gu", dev)
    m.nvfp4_quantize_tile_t(w5, codes=cw, block_scales=sw, codes_t=cwt, block_scales_t=swt, gscales=Sw)
    del w5
    nsets = _copies(cdg.numel() + cwt.numel())
    ops = [(cdg.clone(), cwt.clone()) for _ in range(nsets)]
    out("a6", "nvfp4 DGRAD gate_up (transposed 16x16 copy)", [T5, H5, 2 * I5], _time_rot(torch, [
        (lambda a=a, b=b: m.mx_gemm(m.Operand(m.Format.NVFP4, a, sdg, Sdg, gs=m.GScale.PER_ROW),
                                    m.Operand(m.Format.NVFP4, b, swt, Sw, block=m.Block.TILE, gs=m.GScale.PER_TENSOR),
                                    T5, H5, 2 * I5, out=dx5)) for a, b in ops], 4),
        flops=f, peak=PEAK_F16_TFLOPS, fp4=True, sets=nsets)
    del ops, dx5, cdg, cwt, swt
    ccg, scg, Scg = m.nvfp4_quantize(dyg, block=m.Block.COL, gs=m.GScale.PER_TENSOR, rnd=m.Round.SR, stream_id=1)
    ccx, scx, Scx = m.nvfp4_quantize(x5, block=m.Block.COL, gs=m.GScale.PER_TENSOR)
    del dyg
    dw = torch.empty((2 * I5, H5), dtype=torch.bfloat16, device=dev)
    nsets = _copies(ccg.numel() + ccx.numel())
    ops = [(ccg.clone(), ccx.clone()) for _ in range(nsets)]
    out("a6", "nvfp4 WGRAD gate_up (columnwise copies)", [2 * I5, H5, T5], _time_rot(torch, [
        (lambda a=a, b=b: m.mx_gemm(m.Operand(m.Format.NVFP4, a, scg, Scg, gs=m.GScale.PER_TENSOR),
                                    m.Operand(m.Format.NVFP4, b, scx, Scx, gs=m.GScale.PER_TENSOR),
                                    2 * I5, H5, T5, out=dw)) for a, b in ops], 4),
        flops=f, peak=PEAK_F16_TFLOPS, fp4=True, sets=nsets)
    del x5, dy5, dw, ops, cx, cg, cgc, cw, ccx, ccg
    torch.cuda.empty_cache()

    # ---- Qwen3-8B-shaped dense MLP, MXFP8 (tokens 8192, hidden 4096, I 12288)
    T4, H4, I4 = 8192, 4096, 12288
    x4 = synth.mlp_tensor(4, "x", dev)
    n = T4 * H4
    mc, ms = m.mx_quantize(x4)
    quant_row("a1-a3", "mxfp8 1x32 (X)", x4, lambda xi: lambda: m.mx_quantize(xi, codes=mc, scales=ms),
              n * 2 + n + n // 32)
    d4 = m.mx_quantize(x4, block=m.Block.DUAL)
    quant_row("a1-a3", "mxfp8 dual rowwise + columnwise (X)", x4, lambda xi: lambda: m.mx_quantize(
        xi, block=m.Block.DUAL, codes=d4[0], scales=d4[1], codes_col=d4[2], scales_col=d4[3]),
        n * 2 + 2 * n + 2 * (n // 32))
    w4 = synth.mlp_tensor(4, "w_gu", dev)
    nw = w4.numel()
    wc, wsc = m.mx_quantize(w4, block=m.Block.TILE)
    quant_row("a1-a3", "mxfp8 32x32 (W_gate_up)", w4, lambda xi: lambda: m.mx_quantize(
        xi, block=m.Block.TILE, codes=wc, scales=wsc), nw * 2 + nw + nw // 1024)
    wt4 = m.mx_quantize(w4, block=m.Block.TILE, transposed_copy=True)
    quant_row("a1-a3", "mxfp8 32x32 + transposed copy (W_gate_up)", w4, lambda xi: lambda: m.mx_quantize(
        xi, block=m.Block.TILE, codes=wt4[0], scales=wt4[1], codes_col=wt4[2], scales_col=wt4[3],
        transposed_copy=True), nw * 2 + 2 * nw + 2 * (nw // 1024))
    nsets = _copies(mc.numel())
    mcs = [mc] + [mc.clone() for _ in range(nsets - 1)]
    xo = torch.empty_like(x4)
    out("a4", "mxfp8 dequantize 1x32 -> bf16 (X)", [T4, H4], _time_rot(torch, [
        (lambda c=c: m.mx_dequantize(m.Format.MXFP8, c, ms, T4, H4, out=xo)) for c in mcs], 10),
        nbytes=n + n // 32 + n * 2, sets=nsets)
    del mcs, xo
    y4 = torch.empty((T4, 2 * I4), dtype=torch.bfloat16, device=dev)
    dx4 = torch.empty((T4, H4), dtype=torch.bfloat16, device=dev)
    dw4 = torch.empty((2 * I4, H4), dtype=torch.bfloat16, device=dev)
    f = 2.0 * T4 * 2 * I4 * H4
    dyg4 = synth.mlp_tensor(4, "dy_gu", dev)
    dd = m.mx_quantize(dyg4, block=m.Block.DUAL)

    def gemm_row(row, what, shape, a_ops, b_ops, mnk, outt, fmt, peak, a_kw=None, b_kw=None, iters=5):
        nsets = _copies(a_ops[0].numel() + b_ops[0].numel())
        sets = [(a_ops[0].clone(), b_ops[0].clone()) for _ in range(nsets)]
        fns = [(lambda a=a, b=b: m.mx_gemm(m.Operand(fmt, a, a_ops[1], **(a_kw or {})),
                                           m.Operand(fmt, b, b_ops[1], **(b_kw or {})), *mnk, out=outt))
               for a, b in sets]
        out(row, what, shape, _time_rot(torch, fns, iters), flops=f, peak=peak, sets=nsets)

    MX = m.Format.MXFP8
    gemm_row("a5", "mxfp8 FPROP gate_up", [T4, 2 * I4, H4], (mc, ms), (wc, wsc), (T4, 2 * I4, H4), y4, MX,
             PEAK_FP8_TFLOPS, b_kw=dict(block=m.Block.TILE))
    gemm_row("a5", "mxfp8 DGRAD gate_up (32x32 weight read transposed)", [T4, H4, 2 * I4], (dd[0], dd[1]),
             (wc, wsc), (T4, H4, 2 * I4), dx4, MX, PEAK_FP8_TFLOPS, b_kw=dict(block=m.Block.TILE, transposed=True))
    gemm_row("a5", "mxfp8 DGRAD gate_up (transposed 32x32 copy)", [T4, H4, 2 * I4], (dd[0], dd[1]),
             (wt4[2], wt4[3]), (T4, H4, 2 * I4), dx4, MX, PEAK_FP8_TFLOPS, b_kw=dict(block=m.Block.TILE))
    gemm_row("a5", "mxfp8 WGRAD gate_up (columnwise copies)", [2 * I4, H4, T4], (dd[2], dd[3]), (d4[2], d4[3]),
             (2 * I4, H4, T4), dw4, MX, PEAK_FP8_TFLOPS)
    # the down linear: H [8192, 12288] -> [8192, 4096]
    h4 = synth.mlp_tensor(4, "h", dev)
    wd4 = synth.mlp_tensor(4, "w_dn", dev)
    dyd4 = synth.mlp_tensor(4, "dy_dn", dev)
    hq = m.mx_quantize(h4, block=m.Block.DUAL)
    wdq4 = m.mx_quantize(wd4, block=m.Block.TILE, transposed_copy=True)
    ddq = m.mx_quantize(dyd4, block=m.Block.DUAL)
    del h4, wd4, dyd4
    yd4 = torch.empty((T4, H4), dtype=torch.bfloat16, device=dev)
    dhd4 = torch.empty((T4, I4), dtype=torch.bfloat16, device=dev)
    dwd4 = torch.empty((H4, I4), dtype=torch.bfloat16, device=dev)
    f = 2.0 * T4 * H4 * I4
    gemm_row("a5", "mxfp8 FPROP down", [T4, H4, I4], (hq[0], hq[1]), (wdq4[0], wdq4[1]), (T4, H4, I4), yd4, MX,
             PEAK_FP8_TFLOPS, b_kw=dict(block=m.Block.TILE))
    gemm_row("a5", "mxfp8 DGRAD down (transposed 32x32 copy)", [T4, I4, H4], (ddq[0], ddq[1]), (wdq4[2], wdq4[3]),
             (T4, I4, H4), dhd4, MX, PEAK_FP8_TFLOPS, b_kw=dict(block=m.Block.TILE))
    gemm_row("a5", "mxfp8 WGRAD down (columnwise copies)", [H4, I4, T4], (ddq[2], ddq[3]), (hq[2], hq[3]),
             (H4, I4, T4), dwd4, MX, PEAK_FP8_TFLOPS)
    del hq, wdq4, ddq, yd4, dhd4, dwd4
    f = 2.0 * T4 * 2 * I4 * H4
    # the same layer with DeepSeek-style blockwise FP8 (1x128 / 128x128)
    for f32s in (False, True):
        q = m.fp8bw_quantize_f32 if f32s else m.fp8bw_quantize
        F8 = m.Format.FP8_B128_F32 if f32s else m.Format.FP8_B128
        tag = "f32-scale " if f32s else ""
        sb = 4 if f32s else 1
        b4 = q(x4, block=m.Block.DUAL)
        quant_row("f4", f"fp8 blockwise {tag}dual 1x128 + 128x1 (X)", x4, lambda xi: lambda: q(
            xi, block=m.Block.DUAL, codes=b4[0], scales=b4[1], codes_col=b4[2], scales_col=b4[3]),
            n * 2 + 2 * n + 2 * sb * (n // 128))
        bw4 = q(w4, block=m.Block.TILE, transposed_copy=True)
        quant_row("f4", f"fp8 blockwise {tag}128x128 + transposed copy (W_gate_up)", w4, lambda xi: lambda: q(
            xi, block=m.Block.TILE, codes=bw4[0], scales=bw4[1], codes_col=bw4[2], scales_col=bw4[3],
            transposed_copy=True), nw * 2 + 2 * nw + 2 * sb * (nw // 16384))
        bd = q(dyg4, block=m.Block.DUAL)
        gemm_row("f4", f"fp8 blockwise {tag}FPROP gate_up", [T4, 2 * I4, H4], (b4[0], b4[1]), (bw4[0], bw4[1]),
                 (T4, 2 * I4, H4), y4, F8, PEAK_FP8_TFLOPS, b_kw=dict(block=m.Block.TILE))
        gemm_row("f4", f"fp8 blockwise {tag}DGRAD gate_up (transposed 128x128 copy)", [T4, H4, 2 * I4],
                 (bd[0], bd[1]), (bw4[2], bw4[3]), (T4, H4, 2 * I4), dx4, F8, PEAK_FP8_TFLOPS,
                 b_kw=dict(block=m.Block.TILE))
        gemm_row("f4", f"fp8 blockwise {tag}WGRAD gate_up (columnwise copies)", [2 * I4, H4, T4], (bd[2], bd[3]),
                 (b4[2], b4[3]), (2 * I4, H4, T4), dw4, F8, PEAK_FP8_TFLOPS)
        del b4, bw4, bd
    del x4, w4, wt4, dyg4, dd, d4, y4, dx4, dw4
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

    x3 = bfd(d["x"])
    cx3, sx3, Sx3 = m.nvfp4_quantize(x3)
    wgu = bfd(d["w_gu"].reshape(E * N2, H3)).view(E, N2, H3)
    wdn = bfd(d["w_dn"].reshape(E * H3, I3)).view(E, H3, I3)
    cgu = torch.empty((E, N2, H3 // 2), dtype=torch.uint8, device=dev)
    sgu = torch.empty((E, N2, H3 // 16), dtype=torch.uint8, device=dev)
    Sgu = torch.empty(E, dtype=torch.float32, device=dev)
    cdn = torch.empty((E, H3, I3 // 2), dtype=torch.uint8, device=dev)
    sdn = torch.empty((E, H3, I3 // 16), dtype=torch.uint8, device=dev)
    Sdn = torch.empty(E, dtype=torch.float32, device=dev)
    # expert weights with their scales in the MFMA layout: one 128-byte line
    # holds a stage's scale words of 32 weight rows (the fused Q(H) kernel
    # reads 32-byte row pieces per stage and is bound by L2 requests: 1.18 ms
    # with linear scales, 0.90 ms with these; the other GEMMs run the same)
    L3 = m.Layout.MFMA
    for e in range(E):
        m.nvfp4_quantize(wgu[e], gs=m.GScale.PER_TENSOR, codes=cgu[e], block_scales=sgu[e], gscales=Sgu[e:e + 1],
                         layout=L3)
        m.nvfp4_quantize(wdn[e], gs=m.GScale.PER_TENSOR, codes=cdn[e], block_scales=sdn[e], gscales=Sdn[e:e + 1],
                         layout=L3)
    off_d = torch.from_numpy(off).to(dev)
    idx_d = torch.from_numpy(row_token).to(dev)
    nsets = _copies(cgu.numel())                                   # the 201 MB of NVFP4 gate_up weights
    wsets = [cgu] + [cgu.clone() for _ in range(nsets - 1)]
    A = m.Operand(m.Format.NVFP4, cx3, sx3, Sx3, gs=m.GScale.PER_ROW)
    gu = torch.empty((Mr, N2), dtype=torch.bfloat16, device=dev)
    Bs = [m.Operand(m.Format.NVFP4, w.view(E * N2, H3 // 2), sgu, Sgu, gs=m.GScale.PER_TENSOR, layout=L3)
          for w in wsets]
    out("a8", "MoE grouped gate_up (row gather, 128 experts)", [Mr, N2, H3], _time_rot(torch, [
        (lambda B=B: m.mx_gemm(A, B, Mr, N2, H3, out=gu, group_row_offsets=off_d, a_row_index=idx_d, a_rows=T3))
        for B in Bs], 10), flops=2.0 * Mr * N2 * H3, peak=PEAK_F16_TFLOPS, sets=nsets)
    h = torch.empty((Mr, I3), dtype=torch.bfloat16, device=dev)
    nsets_g = _copies(gu.numel() * 2)
    gus = [gu] + [gu.clone() for _ in range(nsets_g - 1)]
    out("a8", "MoE SwiGLU", [Mr, I3], _time_rot(torch, [(lambda g=g: m.mx_swiglu(g, I3, out=h)) for g in gus], 10),
        nbytes=Mr * N2 * 2 + Mr * I3 * 2, sets=nsets_g)
    del gus
    hf = torch.empty_like(h)
    out("f3", "MoE grouped gate_up with SwiGLU in the epilogue (writes H)", [Mr, N2, H3], _time_rot(torch, [
        (lambda B=B: m.mx_gemm_swiglu(A, B, Mr, I3, H3, out=hf, group_row_offsets=off_d, a_row_index=idx_d,
                                      a_rows=T3)) for B in Bs], 10),
        flops=2.0 * Mr * N2 * H3, peak=PEAK_F16_TFLOPS, sets=nsets)
    cq = torch.empty((Mr, I3 // 2), dtype=torch.uint8, device=dev)
    sq = torch.empty((Mr * (I3 // 16),), dtype=torch.uint8, device=dev)
    Sq = torch.empty((Mr,), dtype=torch.float32, device=dev)
    out("f3", "MoE grouped gate_up with SwiGLU and per-token Q(H) in the epilogue (writes Q(H))", [Mr, N2, H3],
        _time_rot(torch, [(lambda B=B: m.mx_gemm_swiglu_nvfp4(
            A, B, Mr, I3, H3, group_row_offsets=off_d, a_row_index=idx_d, a_rows=T3, codes=cq, block_scales=sq,
            gscales=Sq)) for B in Bs], 10),
        flops=2.0 * Mr * N2 * H3, peak=PEAK_F16_TFLOPS, sets=nsets)
    del hf, Bs, wsets, cq, sq, Sq
    ch, sh, Sh = m.nvfp4_quantize(h)
    quant_row("a8", "MoE per-token Q(H)", h, lambda xi: lambda: m.nvfp4_quantize(
        xi, codes=ch, block_scales=sh, gscales=Sh), Mr * I3 * 2 + Mr * I3 // 2 + Mr * I3 // 16 + Mr * 4)
    y3 = torch.empty((Mr, H3), dtype=torch.bfloat16, device=dev)
    nsets = _copies(cdn.numel())
    Bs = [m.Operand(m.Format.NVFP4, w.view(E * H3, I3 // 2), sdn, Sdn, gs=m.GScale.PER_TENSOR, layout=L3)
          for w in [cdn] + [cdn.clone() for _ in range(nsets - 1)]]
    Ah = m.Operand(m.Format.NVFP4, ch, sh, Sh, gs=m.GScale.PER_ROW)
    out("a8", "MoE grouped down", [Mr, H3, I3], _time_rot(torch, [
        (lambda B=B: m.mx_gemm(Ah, B, Mr, H3, I3, out=y3, group_row_offsets=off_d)) for B in Bs], 10),
        flops=2.0 * Mr * H3 * I3, peak=PEAK_F16_TFLOPS, sets=nsets)


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time bound for the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip the device-copy and host-call probes and the second configuration "
                         "(keeps traced and counted runs to the step)")
    ap.add_argument("--rows", action="store_true",
                    help="only time each hot-path row at the configurations' shapes "
                         "(one JSON line per measurement)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy of known size (counter calibration)")
    ap.add_argument("--oracle-rates", action="store_true",
                    help="only time the CPU oracle per configuration on this host (no GPU)")
    args = ap.parse_args()
    if args.oracle_rates:
        oracle_rates()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(the quantizers shard by rows with no exchange; see the design notes). "
              f"Asked for --gpus {args.gpus} (WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import microscaling_quantization_block_amd as m
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
    log("generating synthetic inputs (seeded, on the device)")
    b = make_buffers(m, torch)
    st = stages(m, b)
    torch.cuda.synchronize()

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        for _, fn, _, _ in st:
            fn()
    torch.cuda.synchronize()

    # the timed steps: back-to-back launches on one stream (torch's current
    # stream, which the library launches on), an event pair around every stage
    log(f"timing {args.steps} steps")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(st) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for j, (_, fn, _, _) in enumerate(st):
            ev[i][j].record()
            fn()
        ev[i][-1].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / args.steps * 1e3
    stage_us = [sum(e[j].elapsed_time(e[j + 1]) for e in ev) / args.steps * 1e3 for j in range(len(st))]
    ms_events = sum(e[0].elapsed_time(e[-1]) for e in ev) / args.steps

    kernels = {name: stage_entry(us, nb, fl) for (name, _, nb, fl), us in zip(st, stage_us)}
    dom = max(range(len(st)), key=lambda j: stage_us[j])
    name, _, nb, fl = st[dom]
    us = stage_us[dom]
    how = (f"HIP events on the launch stream around this stage in each of the {args.steps} timed steps "
           "(one launch per step)")
    if fl is not None:
        tf = fl / (us * 1e-6) / 1e12
        roofline = dict(kernel=name, bound="mfma", achieved=round(tf, 1), peak=PEAK_F16_TFLOPS, unit="TFLOP/s",
                        frac=round(tf / PEAK_F16_TFLOPS, 4), traffic=measured_traffic(name),
                        peak_dtype="fp16 (the MFMA the exact NVFP4 dequant-on-load issues)",
                        frac_fp4_peak=round(tf / PEAK_FP4_TFLOPS, 4), fp4_peak=PEAK_FP4_TFLOPS,
                        us_per_launch=round(us, 1), timing=how)
    else:
        gbps = nb / (us * 1e-6) / 1e9
        roofline = dict(kernel=name, bound="hbm", achieved=round(gbps, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                        frac=round(gbps / PEAK_HBM_GBPS, 4), traffic=measured_traffic(name),
                        us_per_launch=round(us, 1), timing=how)
    value = STEP_FLOPS / (ms_step * 1e-3) / 1e12
    q_us = sum(u for (_, _, nbx, _), u in zip(st, stage_us) if nbx is not None)
    q_bytes = sum(nbx for (_, _, nbx, _) in st if nbx is not None)
    g_us = sum(u for (_, _, _, flx), u in zip(st, stage_us) if flx is not None)
    out = {
        "metric": "MX/NVFP4 quantize GB/s + block-scaled GEMM TFLOP/s (% of gfx950 peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "ms_per_step_events": round(ms_events, 3),
        "launch": "eager (back-to-back launches on one stream)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 (e2m1/e4m3/fp32) -> f16 MFMA, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_mlp_nvfp4_tokens32768_hidden4096_inter14336",
                   "stages": "per linear (gate_up 4096->28672, down 14336->4096): Q(X) rowwise per-token RNE "
                             "and columnwise per-tensor RNE (two passes), Q(W) 16x16 per-tensor RNE with its "
                             "transposed copy, FPROP, Q(dY) rowwise per-token SR and columnwise per-tensor SR "
                             "(two passes), DGRAD (the transposed weight copy), WGRAD",
                   "tokens": T, "hidden": HID, "intermediate": INTER, "seq_len": 8192, "micro_batch": 4,
                   "gemm_tflop_per_step": round(STEP_FLOPS / 1e12, 3)},
        "quantize_GBps": round(q_bytes / (q_us * 1e-6) / 1e9, 1),
        "quantize_frac_hbm": round(q_bytes / (q_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "gemm_TFLOPs": round(STEP_FLOPS / (g_us * 1e-6) / 1e12, 1),
        "gemm_frac_fp16_peak": round(STEP_FLOPS / (g_us * 1e-6) / 1e12 / PEAK_F16_TFLOPS, 4),
        "kernels": kernels,
        "roofline": roofline,
        "config2": None,
        "measured_reference": None,
        "cpu_baseline": None,
    }
    del b, st, ev
    torch.cuda.empty_cache()
    if not args.no_reference:
        log("second configuration (4096 tokens, 2048 -> 768), 200 steps")
        out["config2"] = config2_step(m, torch, 200)
        out["measured_reference"] = measured_reference(m, torch)
    if not args.no_cpu_baseline:
        log(f"CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
