"""GPU parity of the product with Q8_0 weights (mm_mul_mat_q8_0_f32).

Weights are quantized by the oracle (the GPU Q8_0 quantizer's bytes equal
the oracle's, tests/test_gpu_quantize.py); dst must lie within the Q4_0
normwise bound of the oracle's float64 product on every path (the fused
M <= 2 kernel, the tiled int8 MFMA kernel, split-K), and the block dots the
wide kernel writes in its dump mode must equal the oracle's bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import codec, mul_mat
from tests.gpu_util import TOL_Q4_0, assert_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _qs():
    import quantized_skinny_gemm_amd as qs
    return qs


def _debug(wq_dev, x_dev, n, variant, n0, n1):
    """mm_debug_mul_mat on Q8_0 weights: dst and the block dots of columns
    n0..n1-1 (the wide kernel only)."""
    import torch
    qs = _qs()
    m, k = x_dev.shape
    out = torch.empty((m, n), dtype=torch.float32, device=x_dev.device)
    dots = None
    if n1 > n0:
        dots = torch.empty((m, n1 - n0, k // 32), dtype=torch.int32, device=x_dev.device)
    wsb = qs.debug_workspace_size(qs.MM_TYPE_Q8_0, m, n, k, variant)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=x_dev.device)
    st = qs.lib.mm_debug_mul_mat(qs.MM_TYPE_Q8_0, wq_dev.data_ptr(), x_dev.data_ptr(),
                                 out.data_ptr(), None if dots is None else dots.data_ptr(),
                                 m, n, k, n0, n1, variant, ws.data_ptr(), wsb,
                                 torch.cuda.current_stream().cuda_stream)
    return st, out, dots


def _case(m, n, k, seed, scale=0.02):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * scale).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    return codec.quantize_q8_0(w), x


# M = 1, 2 take the fused kernel when K is a multiple of 64 (else the wide
# kernel); larger M the wide kernel (32-, 64- and 128-row tiles, split-K
# when the tiles do not fill the device); ragged N and K.
@pytest.mark.parametrize("m,n,k", [
    (1, 4096, 4096), (2, 11008, 4096), (1, 300, 512), (2, 37, 64), (1, 100, 96), (2, 70, 8224),
    (3, 129, 1024), (8, 250, 2080), (17, 64, 4096), (33, 1000, 512), (64, 200, 1024),
    (130, 33, 8192), (512, 70, 256),
])
def test_q8_0_products(m, n, k):
    qs = _qs()
    wq, x = _case(m, n, k, m * 1_000_003 + n * 17 + k)
    say("q8_0", m, n, k, qs.dispatch(qs.MM_TYPE_Q8_0, m, n, k))
    y = to_host(qs.mul_mat_q8_0_f32(to_dev(wq), to_dev(x)))
    assert_close(y, mul_mat.mul_mat_q8_0_f32(wq, x), TOL_Q4_0, f"q8_0 {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(1, 96, 512), (5, 40, 1024), (40, 130, 2048), (128, 64, 4096)])
def test_q8_0_block_dots_exact(m, n, k):
    """The wide kernel's own int32 block dots equal the oracle's; its dst
    equals the production call's when that call takes the same kernel."""
    import torch
    qs = _qs()
    wq, x = _case(m, n, k, 77 + m + n + k)
    wq_dev, x_dev = to_dev(wq), to_dev(x)
    cols = (0, min(n, 48))
    say("q8_0 dots", m, n, k)
    st, y, dots = _debug(wq_dev, x_dev, n, 2, *cols)
    assert st == 0, qs.status_string(st)
    want = codec.block_dots_q8(wq[cols[0]:cols[1]], codec.quantize_q8_0(x), k)
    assert np.array_equal(to_host(dots), want)
    assert_close(to_host(y), mul_mat.mul_mat_q8_0_f32(wq, x), TOL_Q4_0, "q8_0 wide dump")
    if qs.dispatch(qs.MM_TYPE_Q8_0, m, n, k)[0] == 2:
        assert bool(torch.equal(y, qs.mul_mat_q8_0_f32(wq_dev, x_dev)))


def test_q8_0_extreme_codes_and_scales():
    """Codes at the int8 extremes (-128 included) and scales from a binary16
    subnormal to its largest value: every block dot |S| up to 32 * 128 * 128
    must come out exact, on the fused and on the wide kernel."""
    qs = _qs()
    rng = np.random.default_rng(5)
    n, k = 40, 512
    nb = k // 32
    codes = rng.integers(-128, 128, size=(n, nb, 32))
    codes[0] = -128
    codes[1] = 127
    d_bits = rng.choice(np.array([0x0001, 0x03FF, 0x3C00, 0x7BFF, 0x0400, 0xBC00], dtype=np.uint16),
                        size=(n, nb))
    blk = np.empty((n, nb, 34), dtype=np.uint8)
    blk[..., 0] = d_bits & 0xFF
    blk[..., 1] = d_bits >> 8
    blk[..., 2:] = codes.astype(np.int8).view(np.uint8)
    wq = blk.reshape(n, nb * 34)
    for m in (1, 2, 9):
        x = rng.standard_normal((m, k)).astype(np.float32) * np.float32(1e-3)
        x[0, :32] = -127.0
        ref = mul_mat.mul_mat_q8_0_f32(wq, x)
        say("q8_0 extremes", m)
        y = to_host(qs.mul_mat_q8_0_f32(to_dev(wq), to_dev(x)))
        assert_close(y, ref, TOL_Q4_0, f"q8_0 extremes M={m}")
        st, yw, dots = _debug(to_dev(wq), to_dev(x), n, 2, 0, n)
        assert st == 0, qs.status_string(st)
        assert np.array_equal(to_host(dots), codec.block_dots_q8(wq, codec.quantize_q8_0(x), k))


@pytest.mark.parametrize("j", [0, 1, 2])
def test_q8_0_decode_shapes_and_batch_vs_alone(j):
    """The 7B decode shapes at M = 1 (fused kernel) and a batch whose rows
    equal the rows computed alone within the bound."""
    qs = _qs()
    n, k = workloads.WORKLOADS[1]["shapes"][j]
    w = workloads.weights_f32(workloads.weight_seed(1, j), n, k)
    wq = codec.quantize_q8_0(w)
    wq_dev = to_dev(wq)
    x = workloads.activations(workloads.activation_seed(1, 1), 4, k)
    say("q8_0 decode", n, k)
    ref = mul_mat.mul_mat_q8_0_f32(wq, x)
    full = to_host(qs.mul_mat_q8_0_f32(wq_dev, to_dev(x)))
    assert_close(full, ref, TOL_Q4_0, "q8_0 batch")
    for i in range(4):
        alone = to_host(qs.mul_mat_q8_0_f32(wq_dev, to_dev(x[i:i + 1])))
        assert_close(alone, ref[i:i + 1], TOL_Q4_0, f"q8_0 row {i} alone")


def test_q8_0_debug_rules():
    """The skinny kernel needs K/32 even, and the fused kernel writes no
    block dots: both are argument errors that launch nothing."""
    import torch
    qs = _qs()
    wq, x = _case(1, 64, 512, 9)
    wq_dev, x_dev = to_dev(wq), to_dev(x)
    MM_ERR_ARG = -8
    wq3, x3 = _case(1, 64, 96, 10)
    st, _, _ = _debug(to_dev(wq3), to_dev(x3), 64, 3, 0, 0)
    assert st == MM_ERR_ARG
    st, _, _ = _debug(wq_dev, x_dev, 64, 0, 0, 8)          # M = 1: the fused kernel
    assert st == MM_ERR_ARG
    st, y, _ = _debug(wq_dev, x_dev, 64, 1, 0, 0)           # fused, no dots: fine
    assert st == 0
    torch.cuda.synchronize()
    assert_close(to_host(y), mul_mat.mul_mat_q8_0_f32(wq, x), TOL_Q4_0, "q8_0 forced narrow")


# The skinny kernels on Q8_0 weights (8-, 16- and 32-row passes; 2 < M <= 32
# by default, any M when forced): ragged N, a last phase of fewer than 4
# block pairs (K = 2112: 33 pairs), one pair (K = 64), several passes over M.
@pytest.mark.parametrize("m,n,k", [(3, 300, 512), (8, 4096, 4096), (5, 37, 64), (7, 129, 2112),
                                   (8, 14336, 4096), (20, 100, 1024), (4, 4096, 14336),
                                   (12, 300, 2112), (16, 4096, 4096), (31, 129, 1024),
                                   (32, 1000, 4096), (40, 64, 512)])
def test_q8_0_skinny_products_and_dots(m, n, k):
    import torch
    qs = _qs()
    wq, x = _case(m, n, k, 4000 + m * 31 + n + k)
    wq_dev, x_dev = to_dev(wq), to_dev(x)
    say("q8_0 skinny", m, n, k, qs.dispatch(qs.MM_TYPE_Q8_0, m, n, k))
    cols = (max(0, n - 40), n)
    st, y, dots = _debug(wq_dev, x_dev, n, 3, *cols)
    assert st == 0, qs.status_string(st)
    ref = mul_mat.mul_mat_q8_0_f32(wq, x)
    assert_close(to_host(y), ref, TOL_Q4_0, f"q8_0 skinny {m}x{n}x{k}")
    want = codec.block_dots_q8(wq[cols[0]:cols[1]], codec.quantize_q8_0(x), k)
    assert np.array_equal(to_host(dots), want)
    if qs.dispatch(qs.MM_TYPE_Q8_0, m, n, k)[0] == 3:
        assert bool(torch.equal(y, qs.mul_mat_q8_0_f32(wq_dev, x_dev)))


def test_q8_0_skinny_extremes():
    """Codes -128 and 127 and scales from a binary16 subnormal to its
    largest value through the skinny kernel: exact block dots, dst within
    the bound."""
    qs = _qs()
    rng = np.random.default_rng(6)
    n, k, m = 48, 1024, 6
    nb = k // 32
    codes = rng.integers(-128, 128, size=(n, nb, 32))
    codes[0] = -128
    codes[1] = 127
    d_bits = rng.choice(np.array([0x0001, 0x03FF, 0x3C00, 0x7BFF, 0x0400, 0xBC00], dtype=np.uint16),
                        size=(n, nb))
    blk = np.empty((n, nb, 34), dtype=np.uint8)
    blk[..., 0] = d_bits & 0xFF
    blk[..., 1] = d_bits >> 8
    blk[..., 2:] = codes.astype(np.int8).view(np.uint8)
    wq = blk.reshape(n, nb * 34)
    x = rng.standard_normal((m, k)).astype(np.float32) * np.float32(1e-3)
    x[0, :32] = -127.0
    say("q8_0 skinny extremes")
    st, y, dots = _debug(to_dev(wq), to_dev(x), n, 3, 0, n)
    assert st == 0, qs.status_string(st)
    assert np.array_equal(to_host(dots), codec.block_dots_q8(wq, codec.quantize_q8_0(x), k))
    assert_close(to_host(y), mul_mat.mul_mat_q8_0_f32(wq, x), TOL_Q4_0, "q8_0 skinny extremes")
