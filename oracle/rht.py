"""Random Hadamard transform of the WGRAD inputs, then columnwise NVFP4.

"Train models faster with JAX and MaxText using NVFP4 on NVIDIA Blackwell"
(developer.nvidia.cn), section "NVFP4 pretraining recipe": a random Hadamard
transform is applied to the inputs of the WGRAD GEMM only, to spread outliers
before 4-bit quantization; FPROP and DGRAD skip it, because transforming them
would also transform the weights and break the 16x16 scale consistency.  The
section on enabling NVFP4 in MaxText names the two modes (te_nvfp4 with the
transform, te_nvfp4_no_rht without it).

Readings (the page gives no size, sign rule or arithmetic):

1. The transform runs along the rows, which are the tokens: the contraction
   dimension of WGRAD dW = dY^T X.  It acts on blocks of 16 consecutive rows,
   so each transformed block is exactly one 16x1 block of the columnwise
   NVFP4 copy.
2. Q = (1/4) H16 D, with H16 the Sylvester Hadamard matrix
   H[i][j] = (-1)^popcount(i & j) and D = diag(d), d_i = -1 where bit i of a
   16-bit sign mask is set, else +1.  Q is orthogonal, so when both WGRAD
   operands use the same mask, (Q dY)^T (Q X) = dY^T X before quantization.
   The caller draws the mask (its randomness) and passes it to both.
3. Arithmetic: binary32, d_i * x_i (exact), then the fast Walsh-Hadamard
   butterfly with strides h = 1, 2, 4, 8, each step (u_i, u_{i+h}) <-
   (u_i + u_{i+h}, u_i - u_{i+h}) for every i with i & h == 0, one IEEE
   operation each, then the exact scaling by 1/4.  The quantizer then runs on
   these binary32 values exactly as on any other input (per-tensor second
   scale over the transformed tensor, 16x1 blocks, RNE or SR).

Test infrastructure only (see the package docstring).
"""

import numpy as np

from . import nvfp4

BLOCK = 16
F32 = np.float32


def hadamard16():
    """Sylvester Hadamard matrix of order 16, entries (-1)^popcount(i & j)."""
    i = np.arange(BLOCK)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def signs16(mask):
    """d_i = -1 where bit i of the mask is set, else +1 (float64 [16])."""
    bits = (int(mask) >> np.arange(BLOCK)) & 1
    return np.where(bits == 1, -1.0, 1.0)


def rht16_f64(x, mask):
    """The plain definition in float64: every 16-row block v of every column
    becomes (1/4) H16 (d * v).  x [rows, cols], rows % 16 == 0."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    assert rows % BLOCK == 0
    xb = x.reshape(rows // BLOCK, BLOCK, cols) * signs16(mask)[None, :, None]
    return (np.einsum("ij,bjc->bic", hadamard16(), xb) / 4.0).reshape(rows, cols)


def rht16_f32(x, mask):
    """The same transform in binary32 with the butterfly order of reading 3."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    assert rows % BLOCK == 0
    u = (x.astype(F32).reshape(rows // BLOCK, BLOCK, cols) *
         signs16(mask).astype(F32)[None, :, None]).astype(F32)
    for h in (1, 2, 4, 8):
        nxt = u.copy()
        for i in range(BLOCK):
            if i & h:
                continue
            a, b = u[:, i, :], u[:, i + h, :]
            nxt[:, i, :] = (a + b).astype(F32)
            nxt[:, i + h, :] = (a - b).astype(F32)
        u = nxt
    return (u * F32(0.25)).astype(F32).reshape(rows, cols)


def quantize_colwise_rht(x, mask, gscale="per_tensor", rnd="rne", seed=0, stream_id=1,
                         tensor_tag=0, S_given=None):
    """Columnwise NVFP4 (16x1 blocks along rows, stored transposed, per-tensor
    second scale) of the binary32 transform of x.  Stochastic-rounding draws
    keep the element's index in the [rows, cols] transformed tensor."""
    y = rht16_f32(x, mask).astype(np.float64)
    return nvfp4.quantize_colwise(y, gscale, rnd, seed, stream_id, tensor_tag, S_given)
