"""Pins of oracle/rht.py: the Hadamard matrix against its Kronecker
construction and orthogonality; the binary32 butterfly against the float64
definition (exact on integer inputs, within the rounding bound otherwise);
sign-mask semantics; Q orthogonal, so WGRAD products are unchanged and the
transform inverts; per-block norm preserved; and the quantizer run on the
transformed values (a planted mistake -- a transposed Hadamard order, a lost
sign -- is rejected)."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import nvfp4 as N
from oracle import rht as R


def _bf16(shape, seed, std=1.0):
    x = np.random.default_rng(seed).standard_normal(shape) * std
    return F.bf16_bits_to_f64(F.bf16_rne(x))


def test_hadamard16_is_the_kronecker_power_and_orthogonal():
    h2 = np.array([[1.0, 1.0], [1.0, -1.0]])
    k = h2
    for _ in range(3):
        k = np.kron(k, h2)
    H = R.hadamard16()
    assert np.array_equal(H, k)
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H.T, 16.0 * np.eye(16))
    assert np.all(H[0] == 1.0) and np.all(H[:, 0] == 1.0)


def test_sign_mask_bits():
    assert np.array_equal(R.signs16(0), np.ones(16))
    assert np.array_equal(R.signs16(0xFFFF), -np.ones(16))
    d = R.signs16(0b101)
    assert d[0] == -1 and d[1] == 1 and d[2] == -1 and np.all(d[3:] == 1)


@pytest.mark.parametrize("mask", [0, 0xFFFF, 0x5A3C, 0x0001, 0x8000])
def test_butterfly_equals_definition_on_integers(mask):
    # small integers: every butterfly sum is exact, so binary32 equals float64
    x = np.random.default_rng(mask).integers(-1000, 1000, (64, 24)).astype(np.float64)
    assert np.array_equal(R.rht16_f32(x, mask).astype(np.float64), R.rht16_f64(x, mask))


def test_butterfly_within_rounding_bound_of_definition():
    x = _bf16((256, 40), 1, std=3.0)
    mask = 0xC3A5
    a = R.rht16_f32(x, mask).astype(np.float64)
    b = R.rht16_f64(x, mask)
    # four butterfly stages, each sum rounded once: |err| <= 4 u sum|x_j| / 4
    xs = np.abs(x).reshape(16, 16, 40).sum(axis=1)          # per block and column
    bound = 4 * 2.0 ** -24 * np.repeat(xs, 16, axis=0) / 4 * 1.0001
    assert np.all(np.abs(a - b) <= bound)
    assert np.any(a != b)                                    # real rounding happened


def test_mask_semantics_single_sign_flips_one_input_row():
    x = _bf16((16, 8), 2)
    y0 = R.rht16_f64(x, 0)
    x2 = x.copy()
    x2[5] = -x2[5]
    assert np.allclose(R.rht16_f64(x2, 0), R.rht16_f64(x, 1 << 5), rtol=0, atol=0)
    # the all-ones mask negates the whole transform
    assert np.array_equal(R.rht16_f64(x, 0xFFFF), -y0)


def test_orthogonal_wgrad_product_inverse_and_norm():
    a = _bf16((128, 24), 3)          # dY: tokens x out
    b = _bf16((128, 40), 4)          # X: tokens x in
    mask = 0x9C61
    qa, qb = R.rht16_f64(a, mask), R.rht16_f64(b, mask)
    assert np.allclose(qa.T @ qb, a.T @ b, rtol=1e-12, atol=1e-10)
    # inverse: Q^T = (1/4) D H, i.e. undo the Hadamard then the signs
    H = R.hadamard16()
    back = (np.einsum("ij,bjc->bic", H, qa.reshape(8, 16, 24)) / 4.0) * R.signs16(mask)[None, :, None]
    assert np.allclose(back.reshape(128, 24), a, rtol=0, atol=1e-12)
    na = np.linalg.norm(a.reshape(8, 16, 24), axis=1)
    nq = np.linalg.norm(qa.reshape(8, 16, 24), axis=1)
    assert np.allclose(na, nq, rtol=1e-12)


def test_planted_mistakes_are_rejected():
    x = _bf16((32, 16), 5)
    mask = 0x1234
    y = R.rht16_f64(x, mask)
    # a reversed index order of H (a "transposed" butterfly layout) differs
    Hr = R.hadamard16()[::-1]
    xb = x.reshape(2, 16, 16) * R.signs16(mask)[None, :, None]
    wrong = (np.einsum("ij,bjc->bic", Hr, xb) / 4.0).reshape(32, 16)
    assert not np.allclose(wrong, y)
    # dropping the signs differs
    assert not np.allclose(R.rht16_f64(x, 0), y)


def test_quantize_colwise_rht_runs_the_quantizer_on_the_transform():
    x = _bf16((64, 32), 6)
    mask = 0x00F0
    c, s, S = R.quantize_colwise_rht(x, mask)
    y = R.rht16_f32(x, mask).astype(np.float64)
    c2, s2, S2 = N.quantize_colwise(y)
    assert np.array_equal(c, c2) and np.array_equal(s, s2) and np.array_equal(S, S2)
    # the per-tensor scale comes from the transformed tensor's amax
    assert S[0] == np.float32(np.float32(np.abs(y).max()) / np.float32(2688.0))
    # dequantized transform approximates the transform: the widest E2M1 gap
    # (4 to 6) is two units of the block scale amax_b / 6, E4M3 rounding of
    # that scale adds at most 1/16
    dq = N.dequantize_f64(c, s, S, "1x16", "per_tensor").T
    amax_b = np.repeat(np.abs(y).reshape(4, 16, 32).max(axis=1), 16, axis=0)
    assert np.all(np.abs(dq - y) <= amax_b / 6.0 * (1 + 1 / 16) * 1.001 + 1e-30)
