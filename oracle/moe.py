"""Mixture-of-experts reference: routing, row grouping, and the NVFP4 expert
chain gate_up -> SwiGLU -> per-token requantize -> down.

Miles applies NVFP4 to the routed experts' weights and activations, with a
per-token FP32 activation scale, and quantizes each SwiGLU gate/up pair
together so both halves share one larger scale ("Miles Blackwell RL ...",
sections on the full RL loop and "Um Quantizador Compartilhado É o Verdadeiro
Mecanismo").  Expert weights here use 1x16 blocks along the reduction dim, as
Miles' 1x16 weight layout ("Miles Blackwell RL ...", section on what the Qwen3
ablation does not establish).

Readings (the pages are silent): top-k experts per token by logit (softmax is
monotone, so this equals top-k by probability), ties to the lower expert id;
routed rows are ordered by (expert, token); the combine step (weighted sum of a
token's expert outputs) is not part of this path.  SwiGLU: h = silu(g) * u with
silu(g) = g / (1 + exp(-g)); gate is the first I output columns of gate_up.

Test infrastructure only (see the package docstring).
"""

import numpy as np

from . import nvfp4
from .formats import bf16_rne, bf16_bits_to_f64


def route_topk(logits, k):
    """[T, E] logits -> [T, k] expert ids, best first, ties to the lower id."""
    return np.argsort(-np.asarray(logits, dtype=np.float64), axis=1, kind="stable")[:, :k]


def group_rows(topk, num_experts):
    """Order the (token, expert) pairs by (expert, token).

    Returns (row_token [T*k] int32, group_offsets [E+1] int32)."""
    T, k = topk.shape
    tok = np.repeat(np.arange(T), k)
    exp = topk.reshape(-1)
    order = np.lexsort((tok, exp))
    counts = np.bincount(exp, minlength=num_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return tok[order].astype(np.int32), offsets


def grouped_gemm_f64(a_rows, b_groups, offsets):
    """C[r] = a_rows[r] @ b_groups[g]^T for r in group g (float64)."""
    M = a_rows.shape[0]
    N = b_groups.shape[1]
    out = np.zeros((M, N), dtype=np.float64)
    for g in range(len(offsets) - 1):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            out[lo:hi] = a_rows[lo:hi] @ b_groups[g].T
    return out


def swiglu_f64(gu_bf16_bits, inter):
    """SwiGLU of a [M, 2I] BF16 gate_up output, exact in float64, rounded to BF16."""
    gu = bf16_bits_to_f64(gu_bf16_bits)
    g, u = gu[:, :inter], gu[:, inter:2 * inter]
    h = g / (1.0 + np.exp(-g)) * u
    return bf16_rne(h)


def quantize_expert_weights(w, S_given=None):
    """Per-expert NVFP4 1x16 rowwise copy with one per-tensor S for the whole
    [N, K] expert matrix (for W_gu that is one S over the gate/up pair)."""
    if S_given is None:
        return nvfp4.quantize_rowwise(w, gscale="per_tensor")
    return nvfp4.quantize_rowwise(w, gscale="given", S_given=S_given)
