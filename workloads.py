"""Seeded synthetic inputs shared by the CPU oracle, the GPU tests and the bench.

This module holds no arithmetic of the method itself (no quantisation, no
products): it only draws the random tensors and names the workload shapes, so
that the oracle and the HIP path can be fed the very same host arrays without
sharing any computation.

Workloads stand in for the Llama-7B / Llama-3-8B layer shapes that the pages
talk about (llama.cpp PR 1632, "mulmat tune": all 7B shapes, 4096x4096 Q4_0;
Arm China NUMA article: llama3 Q4_0 MulMat tensors attn_out/ffn_gate/ffn_up/
ffn_out/Q/K/V); no trained weights exist here, so values are drawn i.i.d.:
weights N(0, 0.02) (0.02 read as the standard deviation) and activations
N(0, 1).

Rows are drawn in independent chunks of ``CHUNK_ROWS`` rows, each from its own
generator seeded with ``[seed, chunk]``; any subset of rows can therefore be
regenerated cheaply (the large-shape parity tests sample rows this way).
"""
from __future__ import annotations

import numpy as np

CHUNK_ROWS = 256
WEIGHT_STD = np.float32(0.02)

# (type, [(N, K), ...], [M, ...]) per workload; index = workload id.
WORKLOADS = {
    0: dict(name="tiny_q4_0", types=("q4_0",), shapes=[(256, 512)], ms=[1]),
    1: dict(name="llama7b_decode_q4_0_m1", types=("q4_0",),
            shapes=[(4096, 4096), (11008, 4096), (4096, 11008)], ms=[1]),
    2: dict(name="decode_f16_f32", types=("f16", "f32"),
            shapes=[(4096, 4096), (11008, 4096)], ms=[1, 4, 16]),
    3: dict(name="llama3_8b_ffn_batched_q4_0", types=("q4_0",),
            shapes=[(14336, 4096), (4096, 14336)], ms=[8, 16, 32, 64, 128]),
    4: dict(name="prefill_m512", types=("q4_0", "f16"),
            shapes=[(14336, 4096), (4096, 4096), (128256, 4096)], ms=[512]),
}

# Matrices of one Llama-7B layer at decode (q, k, v, o, gate, up, down).
LLAMA7B_LAYER = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
LLAMA7B_LAYERS = 32


def weight_seed(workload: int, j: int) -> int:
    return 1000 * workload + j


def activation_seed(workload: int, m: int) -> int:
    return 1000 * workload + 500 + m


def _chunk(seed: int, chunk: int, k: int, scale) -> np.ndarray:
    rng = np.random.default_rng([seed, chunk])
    x = rng.standard_normal((CHUNK_ROWS, k), dtype=np.float32)
    if scale is not None:
        x *= scale
    return x


def _rows(seed: int, n: int, k: int, rows, scale) -> np.ndarray:
    if rows is None:
        out = np.empty((n, k), dtype=np.float32)
        for c in range((n + CHUNK_ROWS - 1) // CHUNK_ROWS):
            lo = c * CHUNK_ROWS
            hi = min(n, lo + CHUNK_ROWS)
            out[lo:hi] = _chunk(seed, c, k, scale)[: hi - lo]
        return out
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= n):
        raise IndexError("row index out of range")
    out = np.empty((rows.size, k), dtype=np.float32)
    for c in np.unique(rows // CHUNK_ROWS):
        sel = np.nonzero(rows // CHUNK_ROWS == c)[0]
        out[sel] = _chunk(seed, int(c), k, scale)[rows[sel] - c * CHUNK_ROWS]
    return out


def weights_f32(seed: int, n: int, k: int, rows=None) -> np.ndarray:
    """float32 [n, k] (or the listed rows) drawn N(0, 0.02)."""
    return _rows(seed, n, k, rows, WEIGHT_STD)


def weights_f16(seed: int, n: int, k: int, rows=None) -> np.ndarray:
    """The same draw as ``weights_f32`` stored as binary16 (round to nearest even)."""
    return weights_f32(seed, n, k, rows).astype(np.float16)


def activations(seed: int, m: int, k: int) -> np.ndarray:
    """float32 [m, k] drawn N(0, 1)."""
    return _rows(seed, m, k, None, None)
