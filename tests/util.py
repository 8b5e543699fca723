"""Helpers shared by the tests: device transfer of BF16 bit patterns, GPU
availability, and the library handle.  (Tests may use the oracle; the product
package never does.)"""

import os

import numpy as np
import pytest

try:
    import torch
except Exception:  # pragma: no cover
    torch = None


def gpu_available():
    return torch is not None and torch.cuda.is_available()


requires_gpu = pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")


def to_dev_bf16(bits):
    """numpy uint16 BF16 bit patterns -> CUDA bfloat16 tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def from_dev_bf16(t):
    """CUDA bfloat16 tensor -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_np(t):
    return t.detach().contiguous().cpu().numpy()


def say(msg):
    """Print a progress line that names the case before a GPU step."""
    print(f"[mxq-test] {msg}", flush=True)


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
