"""Writes tests/golden/small_cases.npz from the oracle alone (no GPU code).

Run:  python -m tests.golden.make_golden
The inputs are small seeded BF16 matrices; the outputs are the oracle's codes
and scales for each quantizer mode.  Regenerate only together with a change
to the oracle's arithmetic, naming the passage that justifies it.
"""

import os

import numpy as np

from oracle import mxfp8, nvfp4
from oracle.formats import bf16_rne, bf16_bits_to_f64


def _inputs():
    rs = np.random.default_rng(20261202)
    x = rs.standard_normal((32, 64)) * np.exp(rs.standard_normal((32, 1)))
    x[3, 7] *= 100.0
    x[5, :] = 0.0
    return bf16_bits_to_f64(bf16_rne(x))


def compute():
    x = _inputs()
    out = {"x_bf16": bf16_rne(x)}
    out["mx_row_codes"], out["mx_row_scales"] = mxfp8.quantize_rowwise(x)
    out["mx_col_codes"], out["mx_col_scales"] = mxfp8.quantize_colwise(x)
    out["mx_tile_codes"], out["mx_tile_scales"] = mxfp8.quantize_tile32(x)
    out["nv_row_codes"], out["nv_row_scales"], out["nv_row_S"] = nvfp4.quantize_rowwise(x, "per_row")
    out["nv_sr_codes"], out["nv_sr_scales"], out["nv_sr_S"] = nvfp4.quantize_rowwise(x, "per_row", rnd="sr", seed=0)
    out["nv_col_codes"], out["nv_col_scales"], out["nv_col_S"] = nvfp4.quantize_colwise(x)
    out["nv_tile_codes"], out["nv_tile_scales"], out["nv_tile_S"] = nvfp4.quantize_tile16(x)
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "small_cases.npz")
    np.savez(path, **compute())
    print("wrote", path)
