"""Seeded synthetic inputs shaped like the workloads of the pages.

This module holds input generation only -- none of the quantizers' or GEMMs'
arithmetic -- and serves both the GPU path and the CPU oracle in tests and in
the benchmark.  The pages measure on real models and datasets (Qwen3-30B-A3B
on dapo-math-17k, Qwen3-8B on gsm8k, Llama-3-8B pretraining); these seeded
tensors with the same shapes and stated distributions stand in for them.

Distributions ("N(0, s)" = normal with standard deviation s):
  activations        N(0, 1)
  activations with per-token magnitude   N(0, 1) * exp(N(0, 1)) per row
  weights            N(0, 0.02)
  output gradients   N(0, 1e-3)
  outliers           exactly round(0.001 * n) distinct positions multiplied by
                     100 before BF16 rounding
  router logits      N(0, 1), float32
Values are drawn in float64 (numpy PCG64 on the CPU) or float32 (torch's
generator on a device, for tensors too large to build on the host), then
rounded once to BF16 (round to nearest even).
"""

import numpy as np


def bf16_from_f32(x):
    """float32 array -> BF16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_from_f64(x):
    """float64 -> BF16 bits via one rounding to float32 then one to BF16.

    The float32 step is exact for every value drawn here to within the
    generator's own precision; generation is not part of the method, only its
    result (a BF16 tensor) is."""
    return bf16_from_f32(np.asarray(x, dtype=np.float32))


def rng(seed, tag):
    return np.random.Generator(np.random.PCG64([int(seed), int(tag)]))


def normal_bf16(shape, std, seed, tag):
    return bf16_from_f64(rng(seed, tag).standard_normal(shape) * std)


def token_lognormal_bf16(rows, cols, seed, tag):
    g = rng(seed, tag)
    mag = np.exp(g.standard_normal((rows, 1)))
    return bf16_from_f64(g.standard_normal((rows, cols)) * mag)


def with_outliers_bf16(rows, cols, seed, tag, frac=0.001, factor=100.0):
    g = rng(seed, tag)
    x = g.standard_normal((rows, cols))
    n = rows * cols
    k = int(round(frac * n))
    pos = g.choice(n, size=k, replace=False)
    x.reshape(-1)[pos] *= factor
    return bf16_from_f64(x)


def logits_f32(tokens, experts, seed, tag):
    return rng(seed, tag).standard_normal((tokens, experts)).astype(np.float32)


# ------------------------------------------------------------ workload shapes

CONFIGS = {
    1: dict(name="mxfp8_256x512_gemm256", M=256, K=512, N=256),
    2: dict(name="nvfp4_tok4096_h2048_n768", M=4096, K=2048, N=768),
    3: dict(name="moe_qwen3_30b_a3b_t8192", T=8192, H=2048, E=128, I=768, topk=8),
    4: dict(name="mlp_qwen3_8b_t8192_mxfp8", T=8192, H=4096, I=12288),
    5: dict(name="mlp_llama3_8b_t32768_nvfp4", T=32768, H=4096, I=14336),
}


def config1():
    """MXFP8 1x32 quantize + dequantize of X [256, 512] (N(0,1) with 0.1%
    outliers x100) and a 256x512x256 GEMM against W drawn [K=512, N=256]
    N(0, 0.02), stored [N, K]."""
    x = with_outliers_bf16(256, 512, seed=1, tag=0)
    w_kn = normal_bf16((512, 256), 0.02, seed=1, tag=1)
    w = np.ascontiguousarray(w_kn.T)
    return dict(x=x, w=w)


def config2():
    """NVFP4: X [4096, 2048] N(0,1)*per-token lognormal; W drawn [K=2048, N=768]
    N(0, 0.02) stored [768, 2048]; dY [4096, 768] N(0, 1e-3)."""
    x = token_lognormal_bf16(4096, 2048, seed=2, tag=0)
    w_kn = normal_bf16((2048, 768), 0.02, seed=2, tag=1)
    w = np.ascontiguousarray(w_kn.T)
    dy = normal_bf16((4096, 768), 1e-3, seed=2, tag=2)
    return dict(x=x, w=w, dy=dy)


def config3(tokens=8192, hidden=2048, experts=128, inter=768, topk=8, seed=3):
    """Qwen3-30B-A3B-shaped MoE layer: X [T, H] as in config 2, router logits
    [T, E] N(0,1), W_gu [E, 2I, H] and W_dn [E, H, I] N(0, 0.02)."""
    x = token_lognormal_bf16(tokens, hidden, seed=seed, tag=0)
    logits = logits_f32(tokens, experts, seed=seed, tag=1)
    w_gu = normal_bf16((experts, 2 * inter, hidden), 0.02, seed=seed, tag=2)
    w_dn = normal_bf16((experts, hidden, inter), 0.02, seed=seed, tag=3)
    return dict(x=x, logits=logits, w_gu=w_gu, w_dn=w_dn, topk=topk)


def torch_normal_bf16(shape, std, seed, device):
    """Large tensors: torch's seeded generator on `device`, rounded to BF16.
    (Imported lazily so the CPU-only users of this module need no torch.)"""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
    return t.to(torch.bfloat16)


# Dense-MLP tensors of configurations 4 and 5, generated on the device (shared
# by the benchmark and the full-size parity tests): name -> (shape, std, seed).
def mlp_tensors(cfg):
    c = CONFIGS[cfg]
    T, H, I = c["T"], c["H"], c["I"]
    base = 40 if cfg == 4 else 50
    return {
        "x": ((T, H), 1.0, base + 1),            # gate_up input
        "w_gu": ((2 * I, H), 0.02, base + 3),     # gate_up weight [N, K]
        "dy_gu": ((T, 2 * I), 1e-3, base + 4),    # gate_up output gradient
        "h": ((T, I), 1.0, base + 5),             # down input
        "w_dn": ((H, I), 0.02, base + 6),         # down weight [N, K]
        "dy_dn": ((T, H), 1e-3, base + 7),        # down output gradient
    }


def mlp_tensor(cfg, name, device):
    shape, std, seed = mlp_tensors(cfg)[name]
    return torch_normal_bf16(shape, std, seed, device)
