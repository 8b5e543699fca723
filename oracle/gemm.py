"""Block-scaled GEMM references.

The three GEMMs of a linear layer take quantized inputs and emit BF16
("Train models faster ... NVFP4", section "NVFP4 pretraining recipe":
FPROP, DGRAD and WGRAD with BF16 outputs).  The dequantized backward runs its
GEMMs on BF16 operands equal to DQ(Q(w)) ("NVFP4 RL training", section on the
dequantized backward; "Miles Blackwell RL ...", section on the full RL loop).

A block-scaled GEMM is, up to the order of its sums, the product of the
dequantized operands.  So the reference is that definition:

    C64 = DQ64(A) @ DQ64(B)^T   in float64 (DQ64 = c * s [* S], exact)
    C32 = DQ32(A) @ DQ32(B)^T   in binary32 (BLAS sgemm)

Canonical orientation: C[M, N] = sum_k A[m, k] * B[n, k].

Acceptance (a reading of "BF16-accumulation tolerance"):
    ||C_gpu - C64||_F / ||C64||_F <= 1e-2
    |C_gpu - C32| <= 2^-8 |C32| + K * 2^-23 * (|A| @ |B|^T)      elementwise
The first term covers BF16 output rounding; the second any binary32 summation
order on either side.

Test infrastructure only (see the package docstring).
"""

import numpy as np

from .formats import bf16_bits_to_f64


def gemm_f64(a, b):
    """C = A @ B^T in float64; a [M, K], b [N, K] float64."""
    return np.asarray(a, dtype=np.float64) @ np.asarray(b, dtype=np.float64).T


def gemm_f32(a, b):
    return (np.asarray(a, dtype=np.float32) @ np.asarray(b, dtype=np.float32).T).astype(np.float32)


def abs_product(a, b):
    return np.abs(np.asarray(a, dtype=np.float64)) @ np.abs(np.asarray(b, dtype=np.float64)).T


def rel_frobenius(c_bf16_bits, c64):
    c = bf16_bits_to_f64(c_bf16_bits)
    num = np.linalg.norm(c - c64)
    den = np.linalg.norm(c64)
    return float(num / den) if den > 0 else float(num)


def elementwise_bound(c32, absprod, K):
    return 2.0 ** -8 * np.abs(c32.astype(np.float64)) + K * 2.0 ** -23 * absprod


def check(c_bf16_bits, a_f64, b_f64, a_f32, b_f32, rtol_frob=1e-2):
    """Returns (frobenius error, worst ratio |C_gpu - C32| / bound, ok)."""
    K = a_f64.shape[1]
    c64 = gemm_f64(a_f64, b_f64)
    c32 = gemm_f32(a_f32, b_f32)
    ap = abs_product(a_f64, b_f64)
    c = bf16_bits_to_f64(c_bf16_bits)
    frob = rel_frobenius(c_bf16_bits, c64)
    bound = elementwise_bound(c32, ap, K)
    diff = np.abs(c - c32.astype(np.float64))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, diff / bound, np.where(diff > 0, np.inf, 0.0))
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return frob, worst, (frob <= rtol_frob) and worst <= 1.0
