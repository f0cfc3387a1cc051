"""Pins for the oracle's Q4_0 / Q8_0 codec (CPU only).

Each test ties the oracle to something other than itself: hand-worked bytes
(``tests/golden/blocks.txt``), closed forms evaluated with Python's own
integer / ``struct`` arithmetic, invariants of the definition, exact round
trips of constructed representable blocks, and an exact-rational evaluation
of the fp32 operation sequence at code boundaries.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import codec
from tests.exact import f32, f16, floor_frac, fp16_bits_struct

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "blocks.txt")


def _load_golden():
    cases = []
    cur = None
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                name, typ = rest.split()
                cur = dict(name=name, type=typ)
                cases.append(cur)
            elif key == "x":
                cur["x"] = np.array([float(v) for v in rest.split()], dtype=np.float32)
            elif key == "bytes":
                cur["bytes"] = bytes.fromhex(rest.replace(" ", ""))
    return cases


GOLDEN_CASES = _load_golden()


@pytest.mark.parametrize("case", GOLDEN_CASES, ids=[c["name"] for c in GOLDEN_CASES])
def test_golden_blocks(case):
    x = case["x"].reshape(1, 32)
    assert x.shape == (1, 32)
    if case["type"] == "q4_0":
        assert len(case["bytes"]) == 18
        got = codec.quantize_q4_0(x)
    else:
        assert len(case["bytes"]) == 34
        got = codec.quantize_q8_0(x)
    assert got.tobytes() == case["bytes"], got.tobytes().hex()


def test_golden_negative_zero_in_q8_is_plain_zero():
    got = codec.quantize_q8_0(np.full((1, 32), -0.0, dtype=np.float32))
    assert got.tobytes() == bytes(34)


# ------------------------------------------------------------------ helpers
def _random_blocks(rng, n_blocks):
    """A mix of the workload distribution and harder shapes (spikes, ties, tiny)."""
    parts = [
        rng.standard_normal((n_blocks, 32), dtype=np.float32) * np.float32(0.02),
        rng.standard_normal((n_blocks, 32), dtype=np.float32),
        (rng.integers(-3, 4, size=(n_blocks, 32)) * 0.25).astype(np.float32),
        rng.standard_normal((n_blocks, 32), dtype=np.float32) * np.float32(1e-6),
    ]
    spikes = rng.standard_normal((n_blocks, 32), dtype=np.float32)
    spikes[np.arange(n_blocks), rng.integers(0, 32, n_blocks)] *= np.float32(40)
    parts.append(spikes)
    return np.concatenate(parts).astype(np.float32)


def _signed_absmax_py(block):
    best, mx = 0.0, 0.0
    for v in block:
        if abs(float(v)) > best:
            best, mx = abs(float(v)), float(v)
    return mx


# -------------------------------------------------------------- Q4_0 pins
def test_q4_0_scale_closed_form():
    rng = np.random.default_rng(11)
    x = _random_blocks(rng, 300)
    w = codec.quantize_q4_0(x)
    for i in range(x.shape[0]):
        mx = _signed_absmax_py(x[i])
        d = mx / -8.0                       # exact in binary64
        want = fp16_bits_struct(d)
        got = int(w[i, 0]) | (int(w[i, 1]) << 8)
        if mx == 0.0:
            want = 0x8000                   # -0.0, R3
        assert got == want, (i, mx, hex(got), hex(want))


def test_q4_0_invariants():
    rng = np.random.default_rng(12)
    x = _random_blocks(rng, 2000)
    d32, q = codec.q4_0_codes_fp32(x)
    q = q[:, 0, :]
    d32 = d32[:, 0]
    assert q.min() >= 0 and q.max() <= 15
    idx = np.argmax(np.abs(x), axis=1)
    nz = np.abs(x).max(axis=1) > 0
    # the signed-absmax element lands on code 0 (it maps to -8 d)
    assert np.all(q[np.arange(len(x)), idx][nz] == 0)
    # reconstruction error: |x - d16 (q-8)| <= |d|/2 + 8|d - d16| (+ rounding slack)
    # for elements whose t was not clamped; clamped elements (q = 15) are within |d| + ...
    d16 = codec.fp16_value(codec.fp16_bits(d32)).astype(np.float64)
    xr = d16[:, None] * (q.astype(np.float64) - 8)
    err = np.abs(x.astype(np.float64) - xr)
    ad = np.abs(d32.astype(np.float64))[:, None]
    slack = 8 * np.abs(d32.astype(np.float64) - d16)[:, None] + 1e-6 * ad
    bound = np.where(q == 15, ad, 0.5 * ad) + slack
    assert np.all(err <= bound + 1e-30)


def test_q4_0_representable_round_trip():
    """Blocks built as d16*(q-8) with one element at -8*d16 quantize back to themselves."""
    rng = np.random.default_rng(13)
    for _ in range(300):
        d16 = np.float16(rng.choice([-1, 1]) * rng.uniform(1e-3, 4.0))
        d = np.float32(d16)
        q = rng.integers(1, 16, size=32)
        q[rng.integers(0, 32)] = 0              # the signed absmax element, x = -8 d
        x = (d * (q.astype(np.float32) - 8)).astype(np.float32).reshape(1, 32)
        w = codec.quantize_q4_0(x)
        dd, qq = codec.decode_q4_0(w, 32)
        assert dd[0, 0] == d
        # the first element of largest |x| must be the q=0 element (|q-8| <= 7 elsewhere)
        assert np.array_equal(qq[0, 0], q.astype(np.uint8))
        assert np.array_equal(codec.dequantize_q4_0(w, 32), x)


def test_q4_0_ties_round_up_and_clamp():
    """d a power of two: x = -0.5 d gives t = 8 exactly -> q = 8; x = 7.5 d -> t = 16 -> 15."""
    # max = -8 d (negative) so d > 0 and x/d keeps the sign of x.
    # x/d = -0.5 -> t = 8 -> 8 ; +0.5 -> 9 ; 7.5 -> 16 -> 15 ; -7.5 -> 1 ; 1.5 -> 10 ; -1.5 -> 7
    cases = ((-0.5, 8), (0.5, 9), (7.5, 15), (-7.5, 1), (1.5, 10), (-1.5, 7), (6.49, 14))
    for d in (0.5, 1.0, 2.0, 0.0078125):
        for ratio, want in cases:
            x = np.zeros((1, 32), dtype=np.float32)
            x[0, 0] = -8 * d
            x[0, 5] = ratio * d
            _, q = codec.q4_0_codes_fp32(x)
            assert q[0, 0, 5] == want, (d, ratio)


def _q4_exact_emulation(block):
    """The fp32 op sequence R3-R6 evaluated with exact rationals and explicit rounding."""
    mx = Fraction(_signed_absmax_py(block))
    d = f32(mx / -8)
    idv = f32(1 / d) if d != 0 else Fraction(0)
    out = []
    for v in block:
        p = f32(Fraction(float(v)) * idv)
        t = f32(p + Fraction(17, 2))
        out.append(min(15, max(0, floor_frac(t))))
    return d, out


def _near_boundary_blocks(rng, count):
    """Blocks whose elements sit within a few ulps of a Q4_0 code boundary."""
    blocks = []
    for _ in range(count):
        mx = np.float32(rng.choice([-1, 1]) * rng.uniform(0.01, 3.0))
        d = float(np.float32(mx / np.float32(-8)))
        b = np.zeros(32, dtype=np.float32)
        b[0] = mx
        for j in range(1, 32):
            c = rng.integers(1, 16)
            base = np.float32((c - 8.5) * d)
            b[j] = np.nextafter(base, np.float32(np.inf) * rng.choice([-1, 1]),
                                dtype=np.float32) if rng.random() < 0.5 else base
            for _ in range(int(rng.integers(0, 3))):
                b[j] = np.nextafter(b[j], np.float32(rng.choice([-1, 1]) * np.inf), dtype=np.float32)
        # keep the designated max element the strict absmax
        if np.max(np.abs(b[1:])) >= abs(mx):
            continue
        blocks.append(b)
    return np.array(blocks, dtype=np.float32)


def test_q4_0_matches_exact_rational_fp32_sequence():
    rng = np.random.default_rng(14)
    blocks = _near_boundary_blocks(rng, 400)
    d32, q = codec.q4_0_codes_fp32(blocks)
    differs_from_real = 0
    for i, b in enumerate(blocks):
        d, want = _q4_exact_emulation(b)
        assert Fraction(float(d32[i, 0])) == d
        assert list(q[i, 0]) == want, i
        # count elements where exact-real floor(x/d + 8.5) differs: the test must have teeth
        for j, v in enumerate(b):
            real = min(15, max(0, floor_frac(Fraction(float(v)) / d + Fraction(17, 2)))) if d else 8
            differs_from_real += int(real != want[j])
    assert differs_from_real > 0


# -------------------------------------------------------------- Q8_0 pins
def test_q8_0_scale_closed_form():
    rng = np.random.default_rng(21)
    x = _random_blocks(rng, 300)
    a = codec.quantize_q8_0(x)
    for i in range(x.shape[0]):
        amax = max(abs(float(v)) for v in x[i])
        d = f32(Fraction(amax) / 127)
        want = fp16_bits_struct(float(d))
        got = int(a[i, 0]) | (int(a[i, 1]) << 8)
        assert got == want, (i, amax)


def test_q8_0_invariants():
    rng = np.random.default_rng(22)
    x = _random_blocks(rng, 2000)
    _, q = codec.q8_0_codes_fp32(x)
    q = q[:, 0, :].astype(np.int32)
    assert np.abs(q).max() <= 127
    nz = np.abs(x).max(axis=1) > 0
    idx = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(q[np.arange(len(x)), idx])[nz] == 127)
    assert np.all(q.astype(np.float64) * x.astype(np.float64) >= 0)   # sign preserved


def test_q8_0_representable_round_trip():
    rng = np.random.default_rng(23)
    for _ in range(300):
        q = rng.integers(-127, 128, size=32)
        q[rng.integers(0, 32)] = 127 * rng.choice([-1, 1])
        # d = amax/127 must itself be fp16 so that the round trip is exact: choose d16
        # and set amax = 127 d16; then fl32(amax/127) = d16 exactly.
        d16 = np.float32(np.float16(rng.uniform(1e-3, 2.0)))
        x = (d16 * q.astype(np.float32)).astype(np.float32).reshape(1, 32)
        a = codec.quantize_q8_0(x)
        dd, qq = codec.decode_q8_0(a, 32)
        assert dd[0, 0] == d16
        assert np.array_equal(qq[0, 0].astype(np.int64), q)
        assert np.array_equal(codec.dequantize_q8_0(a, 32), x)


def test_q8_0_matches_exact_rational_fp32_sequence():
    rng = np.random.default_rng(24)
    differs_half_even = 0
    for _ in range(300):
        amax = np.float32(rng.uniform(0.1, 5.0))
        d = f32(Fraction(float(amax)) / 127)
        idv = f32(1 / d)
        b = np.zeros(32, dtype=np.float32)
        b[0] = amax * rng.choice([-1, 1])
        for j in range(1, 32):
            k = rng.integers(0, 127)
            base = np.float32((k + 0.5) * float(d)) * rng.choice([-1, 1])
            for _ in range(int(rng.integers(0, 3))):
                base = np.nextafter(base, np.float32(rng.choice([-1, 1]) * np.inf), dtype=np.float32)
            b[j] = base if abs(base) < amax else 0
        _, q = codec.q8_0_codes_fp32(b.reshape(1, 32))
        for j, v in enumerate(b):
            p = f32(Fraction(float(v)) * idv)
            a = abs(p)
            r = floor_frac(a + Fraction(1, 2))          # half away from zero
            want = r if p >= 0 else -r
            assert int(q[0, 0, j]) == want, (float(v), float(p))
            if a - floor_frac(a) == Fraction(1, 2) and r % 2 == 1:
                differs_half_even += 1
    assert differs_half_even > 0


def test_fp16_conversion_matches_exact_rounding():
    rng = np.random.default_rng(25)
    vals = np.concatenate([
        rng.standard_normal(2000).astype(np.float32) * np.float32(0.01),
        rng.uniform(-7e4, 7e4, 200).astype(np.float32),
        (rng.standard_normal(500) * 1e-6).astype(np.float32),    # fp16 subnormals
        np.float32([6.103515625e-05, 5.960464477539063e-08, 2.98e-08, 65504.0]),
    ])
    vals = vals[np.abs(vals) <= 65504]
    bits = codec.fp16_bits(vals)
    for v, b in zip(vals, bits):
        want = f16(Fraction(float(v)))
        got = Fraction(float(np.uint16(b).view(np.float16)))
        assert got == want, float(v)


def test_k_must_be_multiple_of_block():
    with pytest.raises(ValueError):
        codec.quantize_q4_0(np.zeros((1, 48), dtype=np.float32))
    with pytest.raises(ValueError):
        codec.quantize_q8_0(np.zeros((2, 33), dtype=np.float32))


def test_rows_are_independent():
    """Quantising a row alone or inside a batch gives the same bytes (batch-vs-alone)."""
    rng = np.random.default_rng(26)
    x = rng.standard_normal((7, 256), dtype=np.float32)
    full4, full8 = codec.quantize_q4_0(x), codec.quantize_q8_0(x)
    for i in range(7):
        assert np.array_equal(codec.quantize_q4_0(x[i:i + 1]), full4[i:i + 1])
        assert np.array_equal(codec.quantize_q8_0(x[i:i + 1]), full8[i:i + 1])
