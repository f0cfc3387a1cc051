"""Q4_0 / Q8_0 block codec, step by step in IEEE fp32 (test infrastructure only).

Every step below is one NumPy float32 ufunc call, which is one correctly
rounded IEEE single-precision operation per element; nothing is fused.  The
readings R1-R8 referred to here are listed in the package docstring.

Where the codec sits in the method: llama.cpp PR 1632 "mulmat tune",
Introduction (the quantized MUL_MAT kind, and its INIT stage that converts
``src1``); Arm China NUMA article, MulMat operator section (``src1`` is
quantized into ``wdata`` before the product).
"""
from __future__ import annotations

import numpy as np

QK = 32                  # values per block
Q4_0_BYTES = 18          # fp16 d + 16 bytes of nibbles      (R1)
Q8_0_BYTES = 34          # fp16 d + 32 int8                  (R1)

_F32 = np.float32


def _as_blocks(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("expected a 2-D float32 array [rows, K]")
    rows, k = x.shape
    if k % QK:
        raise ValueError(f"K={k} is not a multiple of {QK}")
    return x.reshape(rows, k // QK, QK)


def fp16_bits(v: np.ndarray) -> np.ndarray:
    """fp32 -> binary16 bit patterns, round to nearest even, subnormals kept (R8)."""
    return np.asarray(v, dtype=np.float32).astype(np.float16).view(np.uint16)


def fp16_value(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns -> their exact value as float32."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def _reciprocal(d: np.ndarray) -> np.ndarray:
    """id = 1/d as one correctly rounded fp32 division, 0 where d == 0 (R5)."""
    safe = np.where(d != 0, d, _F32(1))
    r = (_F32(1) / safe).astype(np.float32)
    return np.where(d != 0, r, _F32(0)).astype(np.float32)


# --------------------------------------------------------------------- Q4_0
def q4_0_signed_absmax(xb: np.ndarray) -> np.ndarray:
    """Per block, the first element with the strictly largest |x| (R3).

    ``argmax`` returns the first index among equal maxima, which is the
    strict-``>`` scan; a block whose |x| are all zero keeps the scan's
    starting value ``+0``.
    """
    a = np.abs(xb)
    idx = np.argmax(a, axis=-1)[..., None]
    amax = np.take_along_axis(a, idx, -1)[..., 0]
    mx = np.take_along_axis(xb, idx, -1)[..., 0]
    return np.where(amax > 0, mx, _F32(0)).astype(np.float32)


def q4_0_codes_fp32(x: np.ndarray):
    """Quantize to Q4_0 codes without packing: returns (d_fp32 [rows, nb], q uint8 [rows, nb, 32]).

    d = max / -8 (fp32; a division by a power of two, so exact unless the
    result is subnormal, where it is the correctly rounded quotient);
    id = 1/d; v = fl32(x*id); t = fl32(v + 8.5); q = clamp(floor(t), 0, 15).
    """
    xb = _as_blocks(x)
    mx = q4_0_signed_absmax(xb)
    d = (mx / _F32(-8)).astype(np.float32)
    idv = _reciprocal(d)
    v = (xb * idv[..., None]).astype(np.float32)          # R5: fp32 product
    t = (v + _F32(8.5)).astype(np.float32)                # R6: fp32 sum
    q = np.clip(np.floor(t), 0, 15).astype(np.uint8)      # R6: floor, clamp
    return d, q


def pack_q4_0(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """(fp32 d [rows, nb], q [rows, nb, 32]) -> uint8 [rows, nb*18] (R1, R2, R8)."""
    rows, nb = d.shape
    out = np.empty((rows, nb, Q4_0_BYTES), dtype=np.uint8)
    out[..., 0:2] = fp16_bits(d).astype("<u2")[..., None].view(np.uint8)
    q = q.astype(np.uint8)
    out[..., 2:] = q[..., :16] | (q[..., 16:] << 4)
    return out.reshape(rows, nb * Q4_0_BYTES)


def quantize_q4_0(x: np.ndarray) -> np.ndarray:
    """float32 [rows, K] -> Q4_0 bytes uint8 [rows, K/32*18]."""
    d, q = q4_0_codes_fp32(x)
    return pack_q4_0(d, q)


def decode_q4_0(w: np.ndarray, k: int):
    """Q4_0 bytes [rows, K/32*18] -> (d as float32 [rows, nb], q uint8 [rows, nb, 32])."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    nb = k // QK
    blk = w.reshape(w.shape[0], nb, Q4_0_BYTES)
    d = fp16_value(blk[..., 0:2].copy().view("<u2")[..., 0])
    qs = blk[..., 2:]
    q = np.concatenate([qs & 0x0F, qs >> 4], axis=-1).astype(np.uint8)
    return d, q


def dequantize_q4_0(w: np.ndarray, k: int) -> np.ndarray:
    """x_hat = f32(d16) * (q - 8); exact in fp32 (11-bit times 4-bit)."""
    d, q = decode_q4_0(w, k)
    x = d[..., None] * (q.astype(np.float32) - _F32(8))
    return x.astype(np.float32).reshape(w.shape[0], k)


# --------------------------------------------------------------------- Q8_0
def q8_0_codes_fp32(x: np.ndarray):
    """Quantize to Q8_0 codes without packing: returns (d_fp32 [rows, nb], q int8 [rows, nb, 32]).

    amax = max |x|; d = fl32(amax / 127); id = 1/d; v = fl32(x*id);
    q = round half away from zero of v (R7), evaluated exactly in float64
    as sign(v) * floor(|v| + 0.5) (|v| + 0.5 is exact in float64 for an
    fp32 v of this range).
    """
    xb = _as_blocks(x)
    amax = np.max(np.abs(xb), axis=-1).astype(np.float32)
    d = (amax / _F32(127)).astype(np.float32)
    idv = _reciprocal(d)
    v = (xb * idv[..., None]).astype(np.float32)
    vd = v.astype(np.float64)
    q = np.sign(vd) * np.floor(np.abs(vd) + 0.5)
    return d, q.astype(np.int8)


def pack_q8_0(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    rows, nb = d.shape
    out = np.empty((rows, nb, Q8_0_BYTES), dtype=np.uint8)
    out[..., 0:2] = fp16_bits(d).astype("<u2")[..., None].view(np.uint8)
    out[..., 2:] = q.astype(np.int8).view(np.uint8)
    return out.reshape(rows, nb * Q8_0_BYTES)


def quantize_q8_0(x: np.ndarray) -> np.ndarray:
    """float32 [rows, K] -> Q8_0 bytes uint8 [rows, K/32*34] (the wdata content)."""
    d, q = q8_0_codes_fp32(x)
    return pack_q8_0(d, q)


def decode_q8_0(a: np.ndarray, k: int):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    nb = k // QK
    blk = a.reshape(a.shape[0], nb, Q8_0_BYTES)
    d = fp16_value(blk[..., 0:2].copy().view("<u2")[..., 0])
    q = blk[..., 2:].copy().view(np.int8)
    return d, q


def dequantize_q8_0(a: np.ndarray, k: int) -> np.ndarray:
    """x_hat = f32(d16) * q; exact in fp32 (11-bit times 8-bit)."""
    d, q = decode_q8_0(a, k)
    return (d[..., None] * q.astype(np.float32)).astype(np.float32).reshape(a.shape[0], k)


# ------------------------------------------------------------ block dots
def block_dots(w_q4: np.ndarray, a_q8: np.ndarray, k: int) -> np.ndarray:
    """S[m, n, b] = sum_j (q4[n,b,j] - 8) * q8[m,b,j] in int64.

    |S| <= 32 * 8 * 127 = 32512, so every value fits int32.
    """
    _, q4 = decode_q4_0(w_q4, k)
    _, q8 = decode_q8_0(a_q8, k)
    w = q4.astype(np.int64) - 8
    a = q8.astype(np.int64)
    return np.einsum("mbj,nbj->mnb", a, w)


def block_dots_q8(w_q8: np.ndarray, a_q8: np.ndarray, k: int) -> np.ndarray:
    """S[m, n, b] = sum_j q8w[n,b,j] * q8a[m,b,j] in int64, for Q8_0 weights.

    |S| <= 32 * 127 * 127 = 516128, so every value fits int32 (and fp32).
    """
    _, qw = decode_q8_0(w_q8, k)
    _, qa = decode_q8_0(a_q8, k)
    return np.einsum("mbj,nbj->mnb", qa.astype(np.int64), qw.astype(np.int64))
