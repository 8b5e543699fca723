"""HIP-graph capture of the hot path: a captured step (per-token NVFP4 Q(X),
per-tensor 16x16 Q(W) with its amax kernels, FPROP, DQ(W), dequantized DGRAD,
plus an MXFP8 DUAL quantization and an SR quantization), on one stream or
with the weight path forked to a second stream, replayed several times, with the program's own eager work and synchronizations between the
replays, must reproduce the eager step's bytes exactly on every replay.  The
library records no memset, so every node is a kernel."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from tests.util import requires_gpu, to_dev_bf16, say

pytestmark = [pytest.mark.gpu, requires_gpu]

M, K, N = 512, 512, 256


def _bf16(shape, std, seed):
    return F.bf16_rne(np.random.default_rng(seed).standard_normal(shape) * std)


def _outputs(dev):
    u8 = dict(dtype=torch.uint8, device=dev)
    return dict(
        cx=torch.empty((M, K // 2), **u8), sx=torch.empty((M, K // 16), **u8),
        Sx=torch.empty(M, dtype=torch.float32, device=dev),
        cw=torch.empty((N, K // 2), **u8), sw=torch.empty((N // 16, K // 16), **u8),
        Sw=torch.empty(1, dtype=torch.float32, device=dev),
        y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
        wdq=torch.empty((N, K), dtype=torch.bfloat16, device=dev),
        dx=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
        mc=torch.empty((M, K), **u8), ms=torch.empty((M, K // 32), **u8),
        mcc=torch.empty((K, M), **u8), msc=torch.empty((K, M // 32), **u8),
        gc=torch.empty((M, N // 2), **u8), gs=torch.empty((M, N // 16), **u8),
        gS=torch.empty(M, dtype=torch.float32, device=dev))


def _step(m, x, w, dy, o):
    m.nvfp4_quantize(x, gs=m.GScale.PER_ROW, codes=o["cx"], block_scales=o["sx"], gscales=o["Sx"])
    m.nvfp4_quantize(w, block=m.Block.TILE, gs=m.GScale.PER_TENSOR, codes=o["cw"],
                     block_scales=o["sw"], gscales=o["Sw"])
    m.mx_gemm(m.Operand(m.Format.NVFP4, o["cx"], o["sx"], o["Sx"], gs=m.GScale.PER_ROW),
              m.Operand(m.Format.NVFP4, o["cw"], o["sw"], o["Sw"], block=m.Block.TILE,
                        gs=m.GScale.PER_TENSOR), M, N, K, out=o["y"])
    m.mx_dequantize(m.Format.NVFP4, o["cw"], o["sw"], N, K, block=m.Block.TILE, gscales=o["Sw"],
                    gs=m.GScale.PER_TENSOR, out=o["wdq"])
    m.mx_gemm(m.Operand(m.Format.BF16, dy, block=m.Block.NONE),
              m.Operand(m.Format.BF16, o["wdq"], block=m.Block.NONE, transposed=True), M, K, N,
              out=o["dx"])
    m.mx_quantize(x, block=m.Block.DUAL, codes=o["mc"], scales=o["ms"], codes_col=o["mcc"],
                  scales_col=o["msc"])
    m.nvfp4_quantize(dy, gs=m.GScale.PER_ROW, rnd=m.Round.SR, seed=7, codes=o["gc"],
                     block_scales=o["gs"], gscales=o["gS"])


def _bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy().copy()


def _step_two_streams(m, x, w, dy, o, side):
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        m.nvfp4_quantize(w, block=m.Block.TILE, gs=m.GScale.PER_TENSOR, codes=o["cw"],
                         block_scales=o["sw"], gscales=o["Sw"])
        done = torch.cuda.Event()
        done.record(side)
        m.mx_dequantize(m.Format.NVFP4, o["cw"], o["sw"], N, K, block=m.Block.TILE, gscales=o["Sw"],
                        gs=m.GScale.PER_TENSOR, out=o["wdq"])
    m.nvfp4_quantize(x, gs=m.GScale.PER_ROW, codes=o["cx"], block_scales=o["sx"], gscales=o["Sx"])
    main.wait_event(done)
    m.mx_gemm(m.Operand(m.Format.NVFP4, o["cx"], o["sx"], o["Sx"], gs=m.GScale.PER_ROW),
              m.Operand(m.Format.NVFP4, o["cw"], o["sw"], o["Sw"], block=m.Block.TILE,
                        gs=m.GScale.PER_TENSOR), M, N, K, out=o["y"])
    main.wait_stream(side)
    m.mx_gemm(m.Operand(m.Format.BF16, dy, block=m.Block.NONE),
              m.Operand(m.Format.BF16, o["wdq"], block=m.Block.NONE, transposed=True), M, K, N,
              out=o["dx"])
    m.mx_quantize(x, block=m.Block.DUAL, codes=o["mc"], scales=o["ms"], codes_col=o["mcc"],
                  scales_col=o["msc"])
    m.nvfp4_quantize(dy, gs=m.GScale.PER_ROW, rnd=m.Round.SR, seed=7, codes=o["gc"],
                     block_scales=o["gs"], gscales=o["gS"])


@pytest.mark.parametrize("two_streams", [False, True])
def test_captured_step_replays_match_eager(two_streams):
    import microscaling_quantization_block_amd as m
    say(f"graph capture of the NVFP4 linear step {M}x{K}x{N}")
    x = to_dev_bf16(_bf16((M, K), 1.0, 1))
    w = to_dev_bf16(_bf16((N, K), 0.02, 2))
    dy = to_dev_bf16(_bf16((M, N), 1e-3, 3))
    eager = _outputs("cuda")
    _step(m, x, w, dy, eager)
    torch.cuda.synchronize()
    want = {k: _bytes(v) for k, v in eager.items()}

    cap = _outputs("cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()                          # default priority
    with torch.cuda.graph(g):
        if two_streams:
            _step_two_streams(m, x, w, dy, cap, side)   # weight path forked to a second stream
        else:
            _step(m, x, w, dy, cap)
    torch.cuda.synchronize()

    other = _outputs("cuda")
    x2 = to_dev_bf16(_bf16((M, K), 3.0, 11))
    for rep in range(4):
        for t in cap.values():
            t.view(torch.uint8).fill_(0xA5)              # stale bytes the replay must overwrite
        _step(m, x2, w, dy, other)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in cap.items():
            got = _bytes(v)
            assert np.array_equal(got, want[k]), f"replay {rep}: {k} differs from the eager step"
