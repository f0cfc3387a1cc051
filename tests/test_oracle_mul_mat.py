"""Pins for the oracle's block dots and float64 products (CPU only).

* block dots: brute force with Python integers, and closed forms;
* Q4_0 product: exact rational evaluation on the tiny 256x512 workload, and
  agreement of two independent formulas (per-block scaled integer sums vs
  DGEMM of the dequantized operands);
* F16 / F32 products: triple loop over Python floats on small shapes;
* row independence (a batch row equals the same row computed alone);
* Q8_0 weights: block dots by brute force and closed forms, the product on
  Q4_0 codes re-encoded as Q8_0 blocks equal to the Q4_0 product, an exact
  rational evaluation from the raw bytes, and the two formulas agreeing.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import workloads
from oracle import codec, mul_mat


def _q4_bytes_from_codes(d16_bits, q):
    """Build Q4_0 bytes directly from codes (bypasses the quantizer)."""
    rows, nb = d16_bits.shape
    out = np.empty((rows, nb, 18), dtype=np.uint8)
    out[..., 0] = d16_bits & 0xFF
    out[..., 1] = d16_bits >> 8
    out[..., 2:] = q[..., :16] | (q[..., 16:] << 4)
    return out.reshape(rows, nb * 18)


def _q8_bytes_from_codes(d16_bits, q):
    rows, nb = d16_bits.shape
    out = np.empty((rows, nb, 34), dtype=np.uint8)
    out[..., 0] = d16_bits & 0xFF
    out[..., 1] = d16_bits >> 8
    out[..., 2:] = q.astype(np.int8).view(np.uint8)
    return out.reshape(rows, nb * 34)


def test_block_dots_closed_forms():
    ones = np.full((1, 1), 0x3C00, dtype=np.uint16)
    q8 = np.full((1, 1, 32), 127, dtype=np.int64)
    a = _q8_bytes_from_codes(ones, q8)
    w0 = _q4_bytes_from_codes(ones, np.zeros((1, 1, 32), dtype=np.uint8))
    w15 = _q4_bytes_from_codes(ones, np.full((1, 1, 32), 15, dtype=np.uint8))
    assert codec.block_dots(w0, a, 32)[0, 0, 0] == -32 * 8 * 127        # -32512
    assert codec.block_dots(w15, a, 32)[0, 0, 0] == 32 * 7 * 127        # 28448
    a_neg = _q8_bytes_from_codes(ones, -q8)
    assert codec.block_dots(w0, a_neg, 32)[0, 0, 0] == 32512


def test_block_dots_brute_force():
    rng = np.random.default_rng(31)
    n, m, nb = 5, 3, 4
    q4 = rng.integers(0, 16, size=(n, nb, 32)).astype(np.uint8)
    q8 = rng.integers(-127, 128, size=(m, nb, 32))
    w = _q4_bytes_from_codes(np.full((n, nb), 0x3C00, dtype=np.uint16), q4)
    a = _q8_bytes_from_codes(np.full((m, nb), 0x3C00, dtype=np.uint16), q8)
    s = codec.block_dots(w, a, nb * 32)
    for i in range(m):
        for j in range(n):
            for b in range(nb):
                want = 0
                for e in range(32):
                    want += (int(q4[j, b, e]) - 8) * int(q8[i, b, e])
                assert s[i, j, b] == want
    # the identity sum(q4*q8) - 8*sum(q8) reaches the same integers
    alt = np.einsum("mbj,nbj->mnb", q8.astype(np.int64), q4.astype(np.int64)) \
        - 8 * q8.astype(np.int64).sum(-1)[:, None, :]
    assert np.array_equal(s, alt)


def test_q4_0_product_exact_rational_tiny_workload():
    """The 256x512 Q4_0 x 1x512 workload, evaluated with exact rationals."""
    w = workloads.weights_f32(workloads.weight_seed(0, 0), 256, 512)
    x = workloads.activations(workloads.activation_seed(0, 1), 1, 512)
    wq = codec.quantize_q4_0(w)
    aq = codec.quantize_q8_0(x)
    got = mul_mat.mul_mat_q4_0_f32(wq, x)
    dw, q4 = codec.decode_q4_0(wq, 512)
    da, q8 = codec.decode_q8_0(aq, 512)
    q4l = q4.astype(int).tolist()
    q8l = q8.astype(int).tolist()
    for n in range(256):
        acc = Fraction(0)
        for b in range(16):
            s = 0
            wr, ar = q4l[n][b], q8l[0][b]
            for e in range(32):
                s += (wr[e] - 8) * ar[e]
            acc += Fraction(float(dw[n, b])) * Fraction(float(da[0, b])) * s
        assert abs(Fraction(float(got[0, n])) - acc) <= abs(acc) * Fraction(1, 10**14) + Fraction(1, 10**300)


def test_q4_0_two_formulas_agree():
    rng = np.random.default_rng(32)
    for (m, n, k) in ((1, 64, 512), (5, 33, 4096), (16, 8, 1024)):
        w = (rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02))
        x = rng.standard_normal((m, k), dtype=np.float32)
        wq = codec.quantize_q4_0(w)
        y1 = mul_mat.mul_mat_q4_0_f32(wq, x)
        y2 = mul_mat.mul_mat_q4_0_f32_dequant(wq, x)
        assert np.max(np.abs(y1 - y2)) <= 1e-12 * np.max(np.abs(y1))


def test_q4_0_product_is_close_to_unquantized():
    """Sanity (not parity): quantized product within a few % of the f32 product."""
    rng = np.random.default_rng(33)
    w = rng.standard_normal((256, 4096), dtype=np.float32) * np.float32(0.02)
    x = rng.standard_normal((4, 4096), dtype=np.float32)
    yq = mul_mat.mul_mat_q4_0_f32(codec.quantize_q4_0(w), x)
    yf = mul_mat.mul_mat_f32(w, x)
    rel = np.linalg.norm(yq - yf) / np.linalg.norm(yf)
    assert 1e-3 < rel < 0.2


def test_f16_f32_products_brute_force():
    rng = np.random.default_rng(34)
    m, n, k = 3, 4, 37
    w = rng.standard_normal((n, k), dtype=np.float32)
    x = rng.standard_normal((m, k), dtype=np.float32)
    wh = w.astype(np.float16)
    y32 = mul_mat.mul_mat_f32(w, x)
    y16 = mul_mat.mul_mat_f16_f32(wh, x)
    for i in range(m):
        for j in range(n):
            s32 = sum(Fraction(float(x[i, e])) * Fraction(float(w[j, e])) for e in range(k))
            s16 = sum(Fraction(float(x[i, e])) * Fraction(float(wh[j, e])) for e in range(k))
            assert abs(Fraction(float(y32[i, j])) - s32) <= Fraction(1, 10**12)
            assert abs(Fraction(float(y16[i, j])) - s16) <= Fraction(1, 10**12)


def test_gemv_is_the_m1_row_of_the_batch():
    """Batch-vs-alone: row m of an M-row product equals the M=1 product of that row."""
    rng = np.random.default_rng(35)
    w = rng.standard_normal((40, 512), dtype=np.float32) * np.float32(0.02)
    x = rng.standard_normal((6, 512), dtype=np.float32)
    wq = codec.quantize_q4_0(w)
    full = mul_mat.mul_mat_q4_0_f32(wq, x)
    for i in range(6):
        assert np.array_equal(mul_mat.mul_mat_q4_0_f32(wq, x[i:i + 1])[0], full[i])


def test_empty_k_is_zero():
    w = np.zeros((3, 0), dtype=np.float32)
    x = np.zeros((2, 0), dtype=np.float32)
    assert np.array_equal(mul_mat.mul_mat_f32(w, x), np.zeros((2, 3)))


# ------------------------------------------------------------ Q8_0 weights
def test_block_dots_q8_closed_forms():
    ones = np.full((1, 1), 0x3C00, dtype=np.uint16)
    top = _q8_bytes_from_codes(ones, np.full((1, 1, 32), 127))
    bottom = _q8_bytes_from_codes(ones, np.full((1, 1, 32), -127))
    most_neg = _q8_bytes_from_codes(ones, np.full((1, 1, 32), -128))
    assert codec.block_dots_q8(top, top, 32)[0, 0, 0] == 32 * 127 * 127          # 516128
    assert codec.block_dots_q8(bottom, top, 32)[0, 0, 0] == -32 * 127 * 127
    assert codec.block_dots_q8(most_neg, top, 32)[0, 0, 0] == -32 * 128 * 127    # the int8 extreme
    assert codec.block_dots_q8(most_neg, most_neg, 32)[0, 0, 0] == 32 * 128 * 128


def test_block_dots_q8_brute_force():
    rng = np.random.default_rng(41)
    n, m, nb = 4, 3, 3
    qw = rng.integers(-128, 128, size=(n, nb, 32))
    qa = rng.integers(-127, 128, size=(m, nb, 32))
    w = _q8_bytes_from_codes(np.full((n, nb), 0x3C00, dtype=np.uint16), qw)
    a = _q8_bytes_from_codes(np.full((m, nb), 0x3C00, dtype=np.uint16), qa)
    s = codec.block_dots_q8(w, a, nb * 32)
    for i in range(m):
        for j in range(n):
            for b in range(nb):
                want = 0
                for e in range(32):
                    want += int(qw[j, b, e]) * int(qa[i, b, e])
                assert s[i, j, b] == want


def test_q8_0_product_on_q4_codes_equals_q4_0_product():
    """Q4_0 weights re-encoded as Q8_0 blocks (same d bits, codes q - 8) give
    the Q4_0 product: the two block types decode to the same values."""
    rng = np.random.default_rng(42)
    for (m, n, k) in ((1, 48, 512), (7, 20, 2048)):
        w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.03)
        x = rng.standard_normal((m, k), dtype=np.float32)
        wq4 = codec.quantize_q4_0(w)
        blk = wq4.reshape(n, k // 32, 18)
        d_bits = blk[..., 0].astype(np.uint16) | (blk[..., 1].astype(np.uint16) << 8)
        codes = np.concatenate([blk[..., 2:] & 15, blk[..., 2:] >> 4], axis=-1).astype(np.int64) - 8
        wq8 = _q8_bytes_from_codes(d_bits, codes)
        y4 = mul_mat.mul_mat_q4_0_f32(wq4, x)
        y8 = mul_mat.mul_mat_q8_0_f32(wq8, x)
        assert np.max(np.abs(y8 - y4)) <= 1e-15 * np.max(np.abs(y4))
        assert np.array_equal(codec.block_dots_q8(wq8, codec.quantize_q8_0(x), k),
                              codec.block_dots(wq4, codec.quantize_q8_0(x), k))


def _f16_exact(lo, hi):
    """Exact value of a little-endian binary16 (two bytes) as a Fraction."""
    bits = int(lo) | (int(hi) << 8)
    sign = -1 if bits >> 15 else 1
    e, f = (bits >> 10) & 31, bits & 1023
    if e == 0:
        return sign * Fraction(f, 1 << 24)
    return sign * Fraction(1024 + f, 1 << 10) * Fraction(2) ** (e - 15)


def test_q8_0_product_exact_rational_from_bytes():
    rng = np.random.default_rng(43)
    m, n, k = 2, 6, 128
    wq8 = codec.quantize_q8_0(rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.05))
    x = rng.standard_normal((m, k), dtype=np.float32)
    aq8 = codec.quantize_q8_0(x)
    got = mul_mat.mul_mat_q8_0_f32(wq8, x)
    wb = wq8.reshape(n, k // 32, 34)
    ab = aq8.reshape(m, k // 32, 34)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for b in range(k // 32):
                s = sum(int(np.int8(wb[j, b, 2 + e])) * int(np.int8(ab[i, b, 2 + e])) for e in range(32))
                acc += _f16_exact(wb[j, b, 0], wb[j, b, 1]) * _f16_exact(ab[i, b, 0], ab[i, b, 1]) * s
            assert abs(Fraction(float(got[i, j])) - acc) <= abs(acc) * Fraction(1, 10**14) + Fraction(1, 10**300)


def test_q8_0_two_formulas_agree():
    rng = np.random.default_rng(44)
    for (m, n, k) in ((1, 64, 512), (5, 33, 4096), (16, 8, 1024)):
        w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
        x = rng.standard_normal((m, k), dtype=np.float32)
        wq = codec.quantize_q8_0(w)
        y1 = mul_mat.mul_mat_q8_0_f32(wq, x)
        y2 = mul_mat.mul_mat_q8_0_f32_dequant(wq, x)
        assert np.max(np.abs(y1 - y2)) <= 1e-12 * np.max(np.abs(y1))
        # and Q8_0 weights sit far closer to the f32 product than Q4_0 ones
        exact = x.astype(np.float64) @ w.astype(np.float64).T
        e8 = np.max(np.abs(y1 - exact))
        e4 = np.max(np.abs(mul_mat.mul_mat_q4_0_f32(codec.quantize_q4_0(w), x) - exact))
        assert e8 < e4

