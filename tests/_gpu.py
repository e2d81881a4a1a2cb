"""Helpers of the GPU tests: moving block arrays between numpy and the device
and the tolerance check.  Nothing here computes any part of the method."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

DEV = "cuda:0"


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy array (structured block arrays become raw bytes) -> device tensor."""
    if a.dtype.names is not None:
        raw = np.ascontiguousarray(a).view(np.uint8).reshape(a.shape[0], -1) if a.ndim >= 1 else \
            np.ascontiguousarray(a).view(np.uint8)
        return torch.from_numpy(raw.copy()).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def blocks_from_dev(t: torch.Tensor, dtype: np.dtype, rows: int) -> np.ndarray:
    raw = t.detach().cpu().numpy().reshape(-1)
    return raw.view(dtype).reshape(rows, -1)


def q81_from_dev(t, rows):
    return blocks_from_dev(t, oracle.Q8_1_DTYPE, rows)


def q80_from_dev(t, rows):
    return blocks_from_dev(t, oracle.Q8_0_DTYPE, rows)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_close(gpu, ref, rel: float, what: str):
    """|gpu - ref| <= rel * max(1, |ref|) elementwise."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bound = rel * np.maximum(1.0, np.abs(ref))
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside {rel}*max(1,|ref|); worst at "
                             f"{i}: gpu {gpu[i]!r} ref {ref[i]!r}")


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                       b.view(torch.int32) if b.dtype == torch.float32 else b)
