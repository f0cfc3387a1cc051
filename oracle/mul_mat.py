"""Reference MUL_MAT products in float64 (test infrastructure only).

``dst[M, N] = src1[M, K] . src0[N, K]^T`` -- llama.cpp PR 1632 "mulmat tune",
Introduction: the three kinds mul_mat_f32 (both F32), mul_mat_f16_f32 (src0
F16) and mul_mat_q_f32 (src0 quantized); Arm China NUMA article, MulMat
operator section: for the quantized kind ``src1`` is first quantized into
``wdata`` and ``dst = src0 * wdata``.

For Q4_0 (and Q8_0 weights) the result that the method reaches is the exact
product of the decoded operands:

    dst[m, n] = sum_b d_w[n, b] * d_a[m, b] * S_b[m, n]

with ``S_b`` the integer block dot (``codec.block_dots``).  Each term is
exact in float64 (11 + 11 + 15 significant bits) and the float64 sum carries
a relative error of about 1e-16, far below the 1e-5 parity bound.
"""
from __future__ import annotations

import numpy as np

from . import codec

_ROW_CHUNK = 2048


def mul_mat_q4_0_f32(w_q4: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Q4_0 src0 bytes [N, K/32*18] x float32 src1 [M, K] -> float64 [M, N].

    INIT: quantize src1 to Q8_0 (the wdata).  COMPUTE: per-block integer
    dots, scaled by both fp16 scales, summed over blocks in float64.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    m, k = x.shape
    a_q8 = codec.quantize_q8_0(x)
    return mul_mat_q4_0_q8_0(w_q4, a_q8, k)


def mul_mat_q4_0_q8_0(w_q4: np.ndarray, a_q8: np.ndarray, k: int) -> np.ndarray:
    """The COMPUTE stage alone: Q4_0 [N, .] x Q8_0 wdata [M, .] -> float64 [M, N]."""
    n = w_q4.shape[0]
    m = a_q8.shape[0]
    da, q8 = codec.decode_q8_0(a_q8, k)
    a = q8.astype(np.int64)
    out = np.empty((m, n), dtype=np.float64)
    for lo in range(0, n, _ROW_CHUNK):
        hi = min(n, lo + _ROW_CHUNK)
        dw, q4 = codec.decode_q4_0(w_q4[lo:hi], k)
        w = q4.astype(np.int64) - 8
        s = np.einsum("mbj,nbj->mnb", a, w)                     # S_b, exact
        scale = da.astype(np.float64)[:, None, :] * dw.astype(np.float64)[None, :, :]
        out[:, lo:hi] = np.sum(scale * s.astype(np.float64), axis=-1)
    return out


def mul_mat_q4_0_f32_dequant(w_q4: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Second, independent formula: DGEMM of the dequantized operands.

    dequant(Q8_0(src1)) @ dequant(Q4_0 src0)^T in float64.  Both operands are
    exact in fp32, so this reaches the same real number as the per-block
    formula, up to float64 summation order.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    k = x.shape[1]
    a = codec.dequantize_q8_0(codec.quantize_q8_0(x), k).astype(np.float64)
    out = np.empty((x.shape[0], w_q4.shape[0]), dtype=np.float64)
    for lo in range(0, w_q4.shape[0], _ROW_CHUNK):
        hi = min(w_q4.shape[0], lo + _ROW_CHUNK)
        w = codec.dequantize_q4_0(w_q4[lo:hi], k).astype(np.float64)
        out[:, lo:hi] = a @ w.T
    return out


def mul_mat_q8_0_f32(w_q8: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Q8_0 src0 bytes [N, K/32*34] x float32 src1 [M, K] -> float64 [M, N].

    The quantized kind with Q8_0 weights (a block type the mulmat tune PR's
    Results section names; its blocks are the ones INIT writes for src1):
    INIT as for Q4_0, then per-block integer dots of the two code sets,
    scaled by both fp16 scales and summed over blocks in float64.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    k = x.shape[1]
    return mul_mat_q8_0_q8_0(w_q8, codec.quantize_q8_0(x), k)


def mul_mat_q8_0_q8_0(w_q8: np.ndarray, a_q8: np.ndarray, k: int) -> np.ndarray:
    """COMPUTE for Q8_0 weights: Q8_0 [N, .] x Q8_0 wdata [M, .] -> float64 [M, N]."""
    n = w_q8.shape[0]
    m = a_q8.shape[0]
    da, qa = codec.decode_q8_0(a_q8, k)
    a = qa.astype(np.int64)
    out = np.empty((m, n), dtype=np.float64)
    for lo in range(0, n, _ROW_CHUNK):
        hi = min(n, lo + _ROW_CHUNK)
        dw, qw = codec.decode_q8_0(w_q8[lo:hi], k)
        s = np.einsum("mbj,nbj->mnb", a, qw.astype(np.int64))   # S_b, exact
        scale = da.astype(np.float64)[:, None, :] * dw.astype(np.float64)[None, :, :]
        out[:, lo:hi] = np.sum(scale * s.astype(np.float64), axis=-1)
    return out


def mul_mat_q8_0_f32_dequant(w_q8: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Second formula for Q8_0 weights: DGEMM of the dequantized operands
    (both exact in fp32), the same real number up to summation order."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    k = x.shape[1]
    a = codec.dequantize_q8_0(codec.quantize_q8_0(x), k).astype(np.float64)
    out = np.empty((x.shape[0], w_q8.shape[0]), dtype=np.float64)
    for lo in range(0, w_q8.shape[0], _ROW_CHUNK):
        hi = min(w_q8.shape[0], lo + _ROW_CHUNK)
        w = codec.dequantize_q8_0(w_q8[lo:hi], k).astype(np.float64)
        out[:, lo:hi] = a @ w.T
    return out


def mul_mat_f16_f32(w_f16: np.ndarray, x: np.ndarray) -> np.ndarray:
    """F16 src0 [N, K] x F32 src1 [M, K] -> float64 [M, N] (no rounding of src1)."""
    w = np.asarray(w_f16, dtype=np.float16).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64) @ w.T


def mul_mat_f32(w_f32: np.ndarray, x: np.ndarray) -> np.ndarray:
    """F32 src0 [N, K] x F32 src1 [M, K] -> float64 [M, N]."""
    w = np.asarray(w_f32, dtype=np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64) @ w.T
