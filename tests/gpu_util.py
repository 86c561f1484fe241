"""Helpers for the GPU parity tests: device copies of host arrays."""
from __future__ import annotations

import numpy as np
import torch

import gguf_quant_dequant_amd as q


def dev():
    return torch.device("cuda", 0)


class DeviceBytes:
    """A host byte array copied to the GPU at a chosen byte offset inside a
    larger allocation (to test 2-byte-aligned weight pointers)."""

    def __init__(self, arr: np.ndarray, offset: int = 0):
        b = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        self.buf = torch.zeros(b.size + offset + 64, dtype=torch.uint8, device=dev())
        self.buf[offset:offset + b.size].copy_(torch.from_numpy(b))
        self.ptr = self.buf.data_ptr() + offset
        self.nbytes = b.size


def run_gemv(fmt, W: np.ndarray, rows: int, cols: int, X: np.ndarray, offset: int = 0):
    Wd = DeviceBytes(W, offset)
    Xd = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).to(dev())
    Y = torch.full((X.shape[0], rows), float("nan"), dtype=torch.float32, device=dev())
    q.qgemv(fmt, Wd.ptr, rows, cols, Xd, Y, X.shape[0])
    torch.cuda.synchronize()
    return Y.cpu().numpy()
