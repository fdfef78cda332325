"""Helpers for the GPU tests: device selection and bit comparisons."""

import math
import struct
import sys

import numpy as np


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no ROCm GPU")
    return torch


def bits(v: float) -> int:
    return struct.unpack("<Q", struct.pack("<d", float(v)))[0]


def same(a: float, b: float) -> bool:
    a, b = float(a), float(b)
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return bits(a) == bits(b)


def say(*args):
    print("[gpu-test]", *args, file=sys.stderr, flush=True)


def to_dev(torch, x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to("cuda")
