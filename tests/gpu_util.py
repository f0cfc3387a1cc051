"""Helpers for the GPU parity tests (imported only by tests marked ``gpu``)."""
from __future__ import annotations

import sys

import numpy as np

# Parity bounds: normwise relative error of the fp32 dst against the float64
# oracle, over the whole matrix and over every row.
TOL_Q4_0 = 1e-5
TOL_F = 1e-3


def say(*args):
    """Name the case before a GPU step, flushed, so a failing run says where it was."""
    print("[gpu-case]", *args, file=sys.stderr, flush=True)


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def normwise_errors(y: np.ndarray, ref: np.ndarray):
    """(matrix error, worst row error): max|y - ref| / max|ref| per matrix and per row."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(y - ref)
    scale = np.max(np.abs(ref))
    mat = float(d.max() / scale) if scale > 0 else float(d.max())
    row_scale = np.max(np.abs(ref), axis=1)
    row_err = np.max(d, axis=1) / np.where(row_scale > 0, row_scale, 1.0)
    return mat, float(row_err.max())


def assert_close(y, ref, tol, what=""):
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    mat, row = normwise_errors(y, ref)
    assert mat <= tol and row <= tol, f"{what}: normwise error {mat:.3e} (row {row:.3e}) > {tol}"
