"""GPU parity with weight matrices larger than 4 GiB.

Every kernel addresses weight rows through byte offsets that pass 2^31 and
2^32 here; a 32-bit product anywhere in the row addressing would read the
wrong rows.  The weights are random bytes made on the device (Q4_0 / Q8_0
blocks with finite binary16 scales of either sign; F16 / F32 values), so no
4 GiB host copy is needed; the oracle computes the sampled output columns
from the same bytes: the first rows, the rows around the 2^31 and 2^32 byte
offsets and the last rows (a ragged tail tile).  Q4_0 also checks the int32
block dots of the last 32 rows bit for bit.  Shapes are chosen so that each
kernel kind the plan has (fused, narrow, skinny MFMA, wide MFMA, each with
its ragged edges) sees such a matrix.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import codec, mul_mat
from tests.gpu_util import TOL_F, TOL_Q4_0, assert_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu

K = 4096


def _qs():
    import quantized_skinny_gemm_amd as qs
    return qs


def _sample_rows(n: int, row_bytes: int) -> np.ndarray:
    picks = [np.arange(0, 8), np.arange(n - 24, n)]
    for off in (1 << 31, 1 << 32):
        r = off // row_bytes
        picks.append(np.arange(max(r - 4, 0), min(r + 4, n)))
    return np.unique(np.concatenate(picks))


def _block_bytes(n: int, nb: int, block: int, seed: int):
    """n x nb random blocks of `block` bytes on the device, bytes 0-1 of each
    a finite binary16 scale in (-0.01, 0.01)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    w = torch.randint(0, 256, (n, nb, block), dtype=torch.uint8, device="cuda", generator=g)
    d = ((torch.rand((n, nb), generator=g, device="cuda") - 0.5) * 0.02).to(torch.float16)
    w[:, :, 0:2] = d.view(torch.uint8).view(n, nb, 2)
    del d
    return w.view(n, nb * block)


def _free():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _check_sampled(y, rows_dev, ref, tol, what):
    """Output columns rows_dev (sampled weight rows) against ref."""
    assert int(rows_dev.max()) < y.shape[1] and ref.shape == (y.shape[0], rows_dev.numel())
    ysel = to_host(y[:, rows_dev])
    assert_close(ysel, ref, tol, what)


def _check_rows(y, rows_dev, ref, tol, what):
    """Output rows rows_dev (sampled src1 rows) against ref."""
    assert int(rows_dev.max()) < y.shape[0] and ref.shape == (rows_dev.numel(), y.shape[1])
    ysel = to_host(y[rows_dev])
    assert_close(ysel, ref, tol, what)


def test_q4_0_and_q8_0_weights_past_4gib():
    import torch
    qs = _qs()
    nb = K // 32
    kinds = set()
    for mm_type, n, block, ms in ((qs.MM_TYPE_Q4_0, 1_900_007, 18, (1, 2, 8, 16, 64, 512)),
                                  (qs.MM_TYPE_Q8_0, 1_000_003, 34, (1, 2, 8, 64))):
        q8 = mm_type == qs.MM_TYPE_Q8_0
        rb = nb * block
        assert n * rb > (1 << 32)
        say("large weights", "q8_0" if q8 else "q4_0", f"N={n} K={K} bytes={n * rb}")
        w = _block_bytes(n, nb, block, 11 + block)
        rows = _sample_rows(n, rb)
        rows_dev = torch.from_numpy(rows).cuda()
        wsel = to_host(w[rows_dev])
        fn = qs.mul_mat_q8_0_f32 if q8 else qs.mul_mat_q4_0_f32
        for m in ms:
            x = workloads.activations(workloads.activation_seed(4, m), m, K)
            disp = qs.dispatch(mm_type, m, n, K)
            kinds.add((mm_type, disp[0]))
            what = f"{'q8_0' if q8 else 'q4_0'} N={n} M={m} dispatch={disp}"
            say("large weights", what)
            y = fn(w, to_dev(x))
            ref = (mul_mat.mul_mat_q8_0_f32_dequant(wsel, x) if q8
                   else mul_mat.mul_mat_q4_0_f32_dequant(wsel, x))
            _check_sampled(y, rows_dev, ref, TOL_Q4_0, what)
            assert bool(torch.isfinite(y).all()), f"{what}: non-finite output"
            del y
            if not q8:
                # the tail rows' block dots, and the forced narrow / wide kernels at M = 8
                for v in ((0, 1, 2) if m == 8 else (0,)):
                    say("large weights dots", what, "variant", v)
                    yd, dots = qs.debug_mul_mat(mm_type, w, to_dev(x), v, n - 32, n)
                    want = codec.block_dots(to_host(w[n - 32:]), codec.quantize_q8_0(x), K)
                    assert np.array_equal(to_host(dots), want), f"{what} variant {v}: block dots"
                    _check_sampled(yd, rows_dev, ref, TOL_Q4_0, f"{what} variant {v}")
                    del yd, dots
            _free()
        if not q8:
            # the same bytes repacked (more than 4 GiB of 16-row tiles): the
            # round trip restores them and the products agree with the oracle
            say("large weights repack", f"N={n}")
            wr = qs.repack_q4_0(w, K)
            assert bool(torch.equal(qs.unpack_q4_0(wr, n, K), w))
            for m in (1, 8, 64):
                x = workloads.activations(workloads.activation_seed(4, m), m, K)
                what = f"q4_0r N={n} M={m} dispatch={qs.dispatch(qs.MM_TYPE_Q4_0R, m, n, K)}"
                say("large weights", what)
                y = qs.mul_mat_q4_0r_f32(wr, n, to_dev(x))
                _check_sampled(y, rows_dev, mul_mat.mul_mat_q4_0_f32_dequant(wsel, x),
                               TOL_Q4_0, what)
                del y
                _free()
            del wr
        del w
        _free()
    # fused / narrow, skinny and wide kernels all saw a matrix past 4 GiB
    assert {(qs.MM_TYPE_Q4_0, 1), (qs.MM_TYPE_Q4_0, 2), (qs.MM_TYPE_Q4_0, 3)} <= kinds
    assert {(qs.MM_TYPE_Q8_0, 1), (qs.MM_TYPE_Q8_0, 2), (qs.MM_TYPE_Q8_0, 3)} <= kinds


@pytest.mark.parametrize("kind", ["f16", "f32"])
def test_f16_f32_weights_past_4gib(kind):
    import torch
    qs = _qs()
    f16 = kind == "f16"
    mm_type = qs.MM_TYPE_F16 if f16 else qs.MM_TYPE_F32
    es = 2 if f16 else 4
    n = (1 << 32) // (K * es) + 37
    assert n * K * es > (1 << 32)
    say("large weights", kind, f"N={n} K={K}")
    g = torch.Generator(device="cuda")
    g.manual_seed(23 + es)
    w = (torch.randn((n, K), generator=g, device="cuda") * 0.02)
    if f16:
        w = w.to(torch.float16)
    _free()
    rows = _sample_rows(n, K * es)
    rows_dev = torch.from_numpy(rows).cuda()
    wsel = to_host(w[rows_dev])
    fn = qs.mul_mat_f16_f32 if f16 else qs.mul_mat_f32
    ref_fn = mul_mat.mul_mat_f16_f32 if f16 else mul_mat.mul_mat_f32
    kinds = set()
    for m in (1, 2, 4, 16, 64):
        x = workloads.activations(workloads.activation_seed(2, m), m, K)
        disp = qs.dispatch(mm_type, m, n, K)
        kinds.add(disp[0])
        what = f"{kind} N={n} M={m} dispatch={disp}"
        say("large weights", what)
        ref = ref_fn(wsel, x)
        y = fn(w, to_dev(x))
        _check_sampled(y, rows_dev, ref, TOL_F, what)
        del y
        if m in (4, 16):
            # the narrow kernel forced, and for F16 the wide one (F32 has none)
            for v in ((1, 2) if f16 else (1,)):
                say("large weights", what, "variant", v)
                yd, _ = qs.debug_mul_mat(mm_type, w, to_dev(x), v)
                _check_sampled(yd, rows_dev, ref, TOL_F, f"{what} variant {v}")
                del yd
        _free()
    assert ({1, 2, 3} if f16 else {1, 3}) <= kinds
    del w
    _free()


@pytest.mark.parametrize("kind", ["f16", "f32"])
def test_tall_f_products_run_over_row_ranges(kind):
    """More than 65535 src1 passes: the narrow and skinny F16 / F32 kernels
    (16-row passes in the grid's y dimension) run as launches over
    consecutive row ranges of 65535 * 16 rows.  Sampled rows on both sides
    of each range boundary and the last rows against the oracle, for the
    kernel the plan picks, each kernel forced, and src1 off its 16-byte
    alignment (the skinny kernel's fallback to the narrow one)."""
    import torch
    qs = _qs()
    f16 = kind == "f16"
    mm_type = qs.MM_TYPE_F16 if f16 else qs.MM_TYPE_F32
    n, k = 40, 64
    span = 65535 * 16
    m = 2 * span + 5
    rng = np.random.default_rng(91 if f16 else 92)
    w = (rng.standard_normal((n, k)) * 0.5).astype(np.float32)
    if f16:
        w = w.astype(np.float16)
    say("tall f products", kind, f"M={m} N={n} K={k}")
    g = torch.Generator(device="cuda")
    g.manual_seed(61)
    xb = torch.randn((m * k + 4,), generator=g, device="cuda")
    x = xb[:m * k].view(m, k)
    xm = xb[1:1 + m * k].view(m, k)                  # the same values shifted by one element
    assert x.data_ptr() % 16 == 0 and xm.data_ptr() % 16 == 4
    rows = np.unique(np.concatenate([np.arange(0, 4), np.arange(span - 8, span + 8),
                                     np.arange(2 * span - 8, m)]))
    rows_dev = torch.from_numpy(rows).cuda()
    ref_fn = mul_mat.mul_mat_f16_f32 if f16 else mul_mat.mul_mat_f32
    ref = ref_fn(w, to_host(x[rows_dev]))
    ref_m = ref_fn(w, to_host(xm[rows_dev]))
    wd = to_dev(w)
    for v in (0, 1, 3):
        what = f"{kind} M={m} variant {v} dispatch={qs.dispatch(mm_type, m, n, k)}"
        say("tall f products", what)
        y, _ = qs.debug_mul_mat(mm_type, wd, x, v)
        _check_rows(y, rows_dev, ref, TOL_F, what)
        assert bool(torch.isfinite(y).all()), f"{what}: non-finite output"
        del y
        _free()
    say("tall f products", kind, "misaligned src1")
    fn = qs.mul_mat_f16_f32 if f16 else qs.mul_mat_f32
    y = fn(wd, xm)
    _check_rows(y, rows_dev, ref_m, TOL_F, f"{kind} misaligned src1")
    assert bool(torch.isfinite(y).all())
    del y, xb, x, xm
    _free()


def _host_blocks(n: int, nb: int, block: int, rng) -> np.ndarray:
    """n x nb random blocks of `block` bytes, bytes 0-1 of each a finite
    binary16 scale in (-0.01, 0.01)."""
    w = rng.integers(0, 256, (n, nb, block), dtype=np.uint8)
    d = ((rng.random((n, nb)) - 0.5) * 0.02).astype(np.float16)
    w[:, :, 0:2] = d.view(np.uint8).reshape(n, nb, 2)
    return w.reshape(n, nb * block)


@pytest.mark.parametrize("kind,k", [("q4_0", 1 << 20), ("q4_0", (1 << 19) + 32),
                                    ("q8_0", 1 << 20), ("q8_0", (1 << 19) + 32),
                                    ("f16", (1 << 20) + 8), ("f32", (1 << 23) + 64)])
def test_long_k(kind, k):
    """K from half a million to past 2^23: the narrow kernel's 16-way K split
    and its reduce, the wide kernel's K split, the skinny kernels' long
    per-wave K runs, an odd block count (K / 32 odd: no block pairs), and for
    F32 past 2^23 the skinny kernel's fallback to the narrow one.  Whole
    outputs against the oracle; Q4_0 block dots of four columns bit for bit."""
    qs = _qs()
    n = 24
    rng = np.random.default_rng(k % 1000 + len(kind))
    ms = (1, 2, 8, 40, 64) if k == (1 << 20) else (1, 8, 64) if k < (1 << 21) else (1, 2, 8)
    if kind in ("q4_0", "q8_0"):
        q8 = kind == "q8_0"
        mm_type = qs.MM_TYPE_Q8_0 if q8 else qs.MM_TYPE_Q4_0
        w = _host_blocks(n, k // 32, 34 if q8 else 18, rng)
        ref_fn = mul_mat.mul_mat_q8_0_f32_dequant if q8 else mul_mat.mul_mat_q4_0_f32_dequant
        fn = qs.mul_mat_q8_0_f32 if q8 else qs.mul_mat_q4_0_f32
        tol = TOL_Q4_0
    else:
        f16 = kind == "f16"
        mm_type = qs.MM_TYPE_F16 if f16 else qs.MM_TYPE_F32
        w = rng.standard_normal((n, k)).astype(np.float16 if f16 else np.float32)
        ref_fn = mul_mat.mul_mat_f16_f32 if f16 else mul_mat.mul_mat_f32
        fn = qs.mul_mat_f16_f32 if f16 else qs.mul_mat_f32
        tol = TOL_F
    wd = to_dev(w)
    for m in ms:
        x = rng.standard_normal((m, k)).astype(np.float32)
        what = f"{kind} M={m} N={n} K={k} dispatch={qs.dispatch(mm_type, m, n, k)}"
        say("long k", what)
        xd = to_dev(x)
        ref = ref_fn(w, x)
        assert_close(to_host(fn(wd, xd)), ref, tol, what)
        if kind == "q4_0":
            say("long k dots", what)
            y, dots = qs.debug_mul_mat(mm_type, wd, xd, 0, n - 4, n)
            assert_close(to_host(y), ref, tol, f"{what} debug")
            want = codec.block_dots(w[n - 4:], codec.quantize_q8_0(x), k)
            assert np.array_equal(to_host(dots), want), f"{what}: block dots"
            del y, dots
        del xd
        _free()
