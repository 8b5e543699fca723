"""The oracle's format constants against the facts the pages state
(tests/golden/format_facts.json, each entry citing its page and section)."""

import json
import os

import numpy as np

from oracle import formats as F
from oracle import mxfp8 as M
from oracle import nvfp4 as N

HERE = os.path.dirname(os.path.abspath(__file__))


def _facts():
    with open(os.path.join(HERE, "golden", "format_facts.json")) as f:
        return json.load(f)


def test_block_sizes_and_formats_follow_the_pages():
    facts = _facts()
    assert M.BLOCK == facts["mxfp8_block_size"]["value"]
    assert N.BLOCK == facts["nvfp4_block_size"]["value"]
    assert facts["nvfp4_weight_block"]["value"] == [N.BLOCK, N.BLOCK]
    assert facts["nvfp4_activation_gradient_block"]["value"] == [1, N.BLOCK]
    # E8M0 carries only an exponent: every finite value is a power of two
    v = F.e8m0_value(np.arange(255))
    assert facts["e8m0_keeps_only_exponent"]["value"]
    assert np.all(np.log2(v) == np.round(np.log2(v)))


def test_golden_regression_fixture():
    """Small fixed-input outputs written by tests/golden/make_golden.py (which
    calls only the oracle): a lock against unintended oracle changes."""
    path = os.path.join(HERE, "golden", "small_cases.npz")
    ref = np.load(path, allow_pickle=False)
    from tests.golden.make_golden import compute
    out = compute()
    assert set(out) == set(ref.files)
    for k in ref.files:
        assert np.array_equal(out[k], ref[k]), k
