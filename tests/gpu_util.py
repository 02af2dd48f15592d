"""Helpers for the GPU parity tests (test code only)."""

from __future__ import annotations

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp8_block_scaled_06_amd as mx
    mx.load_library()          # raises (fails the test) if the library is missing
    return torch


def to_dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda:0")


def to_dev_u8(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda:0")


def to_dev_i32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")


def bf16_host_bits(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu").view(torch.int16).numpy().view(np.uint16)


def u8_host(t) -> np.ndarray:
    return t.detach().to("cpu").numpy()


def log(msg: str):
    print(msg, flush=True)
