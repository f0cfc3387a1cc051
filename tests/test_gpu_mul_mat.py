"""GPU parity of the MUL_MAT kernels against the float64 oracle.

Q4_0: the int32 block dots S_b written by the production kernels must equal
the oracle's exactly; dst must match within 1e-5 normwise (over the matrix
and over each row).  F16 / F32: dst within 1e-3 normwise.  Full outputs are
compared where the oracle finishes in seconds; at the 128256-column prefill
shape, sampled columns (all rows) are compared.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import codec, mul_mat
from tests.gpu_util import TOL_F, TOL_Q4_0, assert_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _qs():
    import quantized_skinny_gemm_amd as qs
    return qs


def _q4_weights(wl, j, n, k):
    """Seeded weights quantized on the GPU; the bytes are checked against the oracle."""
    w = workloads.weights_f32(workloads.weight_seed(wl, j), n, k)
    wq_dev = _qs().quantize_q4_0(to_dev(w))
    wq = codec.quantize_q4_0(w)
    assert np.array_equal(to_host(wq_dev), wq)
    return wq_dev, wq


def _check_q4_product(wq_dev, wq, x, what, variant=0, dots_cols=None):
    qs = _qs()
    m, k = x.shape
    n = wq.shape[0]
    nb = k // 32
    n0, n1 = dots_cols if dots_cols is not None else (0, n)
    say("mul_mat_q4_0", what, f"M={m} N={n} K={k} variant={variant} dots=[{n0},{n1})")
    y, dots = qs.debug_mul_mat(qs.MM_TYPE_Q4_0, wq_dev, to_dev(x), variant, n0, n1)
    y = to_host(y)
    ref = mul_mat.mul_mat_q4_0_f32_dequant(wq, x)
    assert_close(y, ref, TOL_Q4_0, what)
    if dots is not None:
        want = codec.block_dots(wq[n0:n1], codec.quantize_q8_0(x), k)
        got = to_host(dots)
        assert got.shape == (m, n1 - n0, nb)
        assert np.array_equal(got, want), f"{what}: block dots differ"
    return y


def test_tiny_workload_all_paths():
    wq_dev, wq = _q4_weights(0, 0, 256, 512)
    x = workloads.activations(workloads.activation_seed(0, 1), 1, 512)
    y0 = _check_q4_product(wq_dev, wq, x, "tiny auto", 0)
    y1 = _check_q4_product(wq_dev, wq, x, "tiny narrow", 1)
    y2 = _check_q4_product(wq_dev, wq, x, "tiny wide", 2)
    y3 = _check_q4_product(wq_dev, wq, x, "tiny skinny mfma", 3)
    assert np.array_equal(y0, y1)
    # the production entry point gives the same bits as the debug one
    y = to_host(_qs().mul_mat_q4_0_f32(wq_dev, to_dev(x)))
    assert np.array_equal(y, y0)


@pytest.mark.parametrize("j", [0, 1, 2])
def test_llama7b_decode_m1(j):
    n, k = workloads.WORKLOADS[1]["shapes"][j]
    wq_dev, wq = _q4_weights(1, j, n, k)
    x = workloads.activations(workloads.activation_seed(1, 1), 1, k)
    y = _check_q4_product(wq_dev, wq, x, f"7B decode w{j}", 0, (0, n))
    # the production call (fused INIT; one row per wave beyond 8192 rows)
    # gives the same bits as the block-dot dump instantiation
    assert np.array_equal(to_host(_qs().mul_mat_q4_0_f32(wq_dev, to_dev(x))), y)


@pytest.mark.parametrize("j", [0, 1])
def test_llama3_ffn_batched(j):
    n, k = workloads.WORKLOADS[3]["shapes"][j]
    wq_dev, wq = _q4_weights(3, j, n, k)
    for m in workloads.WORKLOADS[3]["ms"]:
        x = workloads.activations(workloads.activation_seed(3, m), m, k)
        cols = (n - 200, n) if m >= 32 else (0, 256)
        _check_q4_product(wq_dev, wq, x, f"ffn w{j} M={m}", 0, cols)


def test_threshold_both_kernels_agree_with_oracle():
    """Around the narrow/wide threshold, both kernels on the same inputs."""
    n, k = 4096, 14336
    wq_dev, wq = _q4_weights(3, 1, n, k)
    for m in (1, 4, 8, 9, 16, 32, 33):
        x = workloads.activations(workloads.activation_seed(3, m), m, k)
        for v in (1, 2, 3):
            _check_q4_product(wq_dev, wq, x, f"threshold M={m}", v, (0, 64))


def _sampled_cols(n, seed, count=384):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(0, 64), np.arange(n - 64, n),
                                     rng.integers(0, n, count)]))


@pytest.mark.parametrize("j", [0, 1, 2])
def test_prefill_m512_q4_0(j):
    import torch
    qs = _qs()
    n, k = workloads.WORKLOADS[4]["shapes"][j]
    seed = workloads.weight_seed(4, j)
    w = workloads.weights_f32(seed, n, k)
    say("prefill q4_0 quantize", j, n, k)
    wq_dev = qs.quantize_q4_0(to_dev(w))
    del w
    x = workloads.activations(workloads.activation_seed(4, 512), 512, k)
    say("prefill q4_0 mul_mat", j)
    cols = _sampled_cols(n, 40 + j)
    y, dots = qs.debug_mul_mat(qs.MM_TYPE_Q4_0, wq_dev, to_dev(x), 0, n - 32, n)
    ysel = to_host(y[:, torch.from_numpy(cols).cuda()])
    wsel = codec.quantize_q4_0(workloads.weights_f32(seed, n, k, rows=cols))
    assert np.array_equal(to_host(wq_dev[torch.from_numpy(cols).cuda()]), wsel)
    ref = mul_mat.mul_mat_q4_0_f32_dequant(wsel, x)
    assert_close(ysel, ref, TOL_Q4_0, f"prefill q4_0 w{j}")
    wtail = codec.quantize_q4_0(workloads.weights_f32(seed, n, k, rows=np.arange(n - 32, n)))
    assert np.array_equal(to_host(dots), codec.block_dots(wtail, codec.quantize_q8_0(x), k))
    # the unsampled columns: every output finite and the production entry gives the same bits
    y2 = qs.mul_mat_q4_0_f32(wq_dev, to_dev(x))
    assert bool(torch.equal(y, y2))
    assert bool(torch.isfinite(y).all())
    del y, y2, wq_dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("j", [0, 1, 2])
def test_prefill_m512_f16(j):
    import torch
    qs = _qs()
    n, k = workloads.WORKLOADS[4]["shapes"][j]
    seed = workloads.weight_seed(4, j)
    say("prefill f16", j, n, k)
    w16 = to_dev(workloads.weights_f16(seed, n, k))
    x = workloads.activations(workloads.activation_seed(4, 512), 512, k)
    y = qs.mul_mat_f16_f32(w16, to_dev(x))
    cols = _sampled_cols(n, 50 + j)
    ysel = to_host(y[:, torch.from_numpy(cols).cuda()])
    ref = mul_mat.mul_mat_f16_f32(workloads.weights_f16(seed, n, k, rows=cols), x)
    assert_close(ysel, ref, TOL_F, f"prefill f16 w{j}")
    del y, w16
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", ["f16", "f32"])
@pytest.mark.parametrize("j", [0, 1])
def test_decode_f16_f32(kind, j):
    qs = _qs()
    n, k = workloads.WORKLOADS[2]["shapes"][j]
    seed = workloads.weight_seed(2, j)
    w = workloads.weights_f16(seed, n, k) if kind == "f16" else workloads.weights_f32(seed, n, k)
    wd = to_dev(w)
    for m in workloads.WORKLOADS[2]["ms"]:
        x = workloads.activations(workloads.activation_seed(2, m), m, k)
        say("decode", kind, j, m)
        fn = qs.mul_mat_f16_f32 if kind == "f16" else qs.mul_mat_f32
        y = to_host(fn(wd, to_dev(x)))
        ref = mul_mat.mul_mat_f16_f32(w, x) if kind == "f16" else mul_mat.mul_mat_f32(w, x)
        assert_close(y, ref, TOL_F, f"{kind} w{j} M={m}")


# ------------------------------------------------------------------ edges
@pytest.mark.parametrize("m,n,k", [
    (1, 1, 32), (1, 1000, 96), (3, 257, 4128), (8, 129, 2080), (9, 77, 1056),
    (16, 300, 544), (33, 65, 3200), (100, 190, 512), (130, 33, 8192), (513, 70, 256),
    (1, 64, 14336), (32, 64, 14336), (2, 7, 32), (100, 8200, 256),
])
def test_ragged_shapes_q4_0(m, n, k):
    rng = np.random.default_rng(m * 1_000_003 + n * 101 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    wq = codec.quantize_q4_0(w)
    wq_dev = to_dev(wq)
    for v in (0, 1, 2, 3):
        _check_q4_product(wq_dev, wq, x, f"ragged {m}x{n}x{k}", v, (0, min(n, 40)))


# The skinny MFMA kernels (2 < M <= 32, K % 64 == 0): a last phase of fewer
# than 4 block pairs, a last wave with a shorter run, a single block pair,
# N off the 16-row workgroup and M off the 8- and 16-row tiles.
@pytest.mark.parametrize("m,n,k", [
    (3, 100, 4160), (5, 17, 64), (7, 333, 1088), (8, 40, 192), (9, 50, 4160),
    (13, 257, 320), (16, 31, 2112), (17, 99, 4160), (31, 65, 576), (32, 48, 128),
])
def test_ragged_shapes_skinny_q4_0(m, n, k):
    qs = _qs()
    assert qs.dispatch(qs.MM_TYPE_Q4_0, m, n, k)[0] == 3
    rng = np.random.default_rng(m * 7_000_003 + n * 131 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    wq = codec.quantize_q4_0(w)
    wq_dev = to_dev(wq)
    y = _check_q4_product(wq_dev, wq, x, f"skinny ragged {m}x{n}x{k}", 0)
    _check_q4_product(wq_dev, wq, x, f"skinny ragged {m}x{n}x{k}", 3)
    # the production instantiation (no block-dot dump) gives the same bits
    assert np.array_equal(to_host(qs.mul_mat_q4_0_f32(wq_dev, to_dev(x))), y)


# The M <= 8 skinny kernel over many row tiles: N off the 16-row tiles, K off
# the phases, waves with no K range (K = 256 is one phase), M below 8.
@pytest.mark.parametrize("m,n,k", [(8, 8192, 4096), (5, 8200, 4160), (1, 8192, 256), (3, 12000, 1088)])
def test_many_tiles_skinny_q4_0(m, n, k):
    qs = _qs()
    if m > 2:
        assert qs.dispatch(qs.MM_TYPE_Q4_0, m, n, k)[0] == 3
    rng = np.random.default_rng(m * 5_000_011 + n * 37 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    wq = codec.quantize_q4_0(w)
    wq_dev = to_dev(wq)
    y = _check_q4_product(wq_dev, wq, x, f"skinny many tiles {m}x{n}x{k}", 3)
    if m > 2:
        assert np.array_equal(to_host(qs.mul_mat_q4_0_f32(wq_dev, to_dev(x))), y)


# M = 2 with long K (one weight row per wave, 16 waves per workgroup in the
# fused kernel): N off the row groups; the production call against the
# oracle and bit for bit against the narrow kernel's dump instantiation.
def test_fused_m2_long_k():
    qs = _qs()
    m, n, k = 2, 4100, 8448
    rng = np.random.default_rng(424242)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    wq = codec.quantize_q4_0(w)
    wq_dev = to_dev(wq)
    y = _check_q4_product(wq_dev, wq, x, "fused M=2 long K", 1, (0, 64))
    assert np.array_equal(to_host(qs.mul_mat_q4_0_f32(wq_dev, to_dev(x))), y)


# The fused kernel quantizes src1 with four lanes per block where that takes
# one round of its threads (8-wave workgroups: K <= 4096 at M = 1, 2048 at
# M = 2), else with two (and always two with 16-wave workgroups, K > 8192):
# on both sides of each bound, the production call against the oracle and
# bit for bit against the narrow kernel's dump instantiation (block dots
# exact), whose codes come from the two-lane routine.
@pytest.mark.parametrize("m,k", [(1, 4096), (1, 4160), (1, 8192), (1, 8256), (1, 11008),
                                 (2, 2048), (2, 2112), (2, 4096)])
def test_fused_src1_lanes_per_block(m, k):
    qs = _qs()
    n = 2100                          # enough rows that K is not split
    rng = np.random.default_rng(1000 * m + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[0, :64] *= 1e-5                 # binary16-subnormal scales in the first blocks
    wq = codec.quantize_q4_0(w)
    wq_dev = to_dev(wq)
    v, split, _, _, launches = qs.dispatch(qs.MM_TYPE_Q4_0, m, n, k)
    assert (v, split, launches) == (1, 1, 1), "the fused kernel, one launch"
    y = _check_q4_product(wq_dev, wq, x, f"fused lanes M={m} K={k}", 1, (0, 300))
    assert np.array_equal(to_host(qs.mul_mat_q4_0_f32(wq_dev, to_dev(x))), y)


def test_misaligned_src0_uses_generic_path():
    """src0 at a 2-byte (not 4-byte) offset: the kernels fall back to 16-bit loads."""
    import torch
    rng = np.random.default_rng(9)
    n, k = 96, 1024
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    wq = codec.quantize_q4_0(w)
    buf = torch.zeros(wq.size + 16, dtype=torch.uint8, device="cuda")
    view = buf[2:2 + wq.size].view(n, wq.shape[1])
    view.copy_(torch.from_numpy(wq).cuda())
    assert view.data_ptr() % 4 == 2
    # M <= 2: the fused kernel needs 4-byte aligned weights, so the general
    # narrow kernel quantizes src1 in LDS instead
    for m in (1, 2, 5):
        x = rng.standard_normal((m, k)).astype(np.float32)
        for v in (0, 1, 2, 3):
            _check_q4_product(view, wq, x, f"misaligned M={m}", v, (0, 8))
        y = to_host(_qs().mul_mat_q4_0_f32(view, to_dev(x)))
        assert_close(y, mul_mat.mul_mat_q4_0_f32_dequant(wq, x), TOL_Q4_0, f"misaligned M={m}")


@pytest.mark.parametrize("m", [5, 40])
def test_misaligned_f16_f32_operands(m):
    """src0 and src1 off their 16-byte alignment (src0 by 2 bytes for F16, by 4 for
    F32; src1 by 4): the skinny MFMA kernel falls back to the narrow one, the wide
    F16 kernel and its src1 conversion take their element-wise paths."""
    import torch
    qs = _qs()
    rng = np.random.default_rng(77 + m)
    n, k = 200, 1024
    w = rng.standard_normal((n, k)).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    wh = w.astype(np.float16)
    say("misaligned f", m, n, k)
    xb = torch.zeros(m * k + 4, dtype=torch.float32, device="cuda")
    xv = xb[1:1 + m * k].view(m, k)
    xv.copy_(torch.from_numpy(x).cuda())
    assert xv.data_ptr() % 16 == 4
    hb = torch.zeros(n * k + 8, dtype=torch.float16, device="cuda")
    hv = hb[1:1 + n * k].view(n, k)
    hv.copy_(torch.from_numpy(wh).cuda())
    assert hv.data_ptr() % 16 == 2
    fb = torch.zeros(n * k + 4, dtype=torch.float32, device="cuda")
    fv = fb[1:1 + n * k].view(n, k)
    fv.copy_(torch.from_numpy(w).cuda())
    assert fv.data_ptr() % 16 == 4
    assert_close(to_host(qs.mul_mat_f16_f32(hv, xv)), mul_mat.mul_mat_f16_f32(wh, x), TOL_F, "f16")
    assert_close(to_host(qs.mul_mat_f32(fv, xv)), mul_mat.mul_mat_f32(w, x), TOL_F, "f32")
    # the wide F16 kernel forced on the same operands: element-wise weight
    # loads (src0 off 16 bytes) and src1 conversion (src1 off 16 bytes)
    y, _ = qs.debug_mul_mat(qs.MM_TYPE_F16, hv, xv, 2)
    assert_close(to_host(y), mul_mat.mul_mat_f16_f32(wh, x), TOL_F, "f16 wide")
    y, _ = qs.debug_mul_mat(qs.MM_TYPE_F16, to_dev(wh), xv, 2)
    assert_close(to_host(y), mul_mat.mul_mat_f16_f32(wh, x), TOL_F, "f16 wide, aligned src0")
    # aligned weights, misaligned src1 only
    assert_close(to_host(qs.mul_mat_f16_f32(to_dev(wh), xv)), mul_mat.mul_mat_f16_f32(wh, x), TOL_F,
                 "f16 aligned src0")
    assert_close(to_host(qs.mul_mat_f32(to_dev(w), xv)), mul_mat.mul_mat_f32(w, x), TOL_F,
                 "f32 aligned src0")


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (2, 33, 7), (5, 100, 1000), (16, 129, 257),
                                   (17, 70, 300), (40, 300, 64), (130, 129, 200)])
def test_ragged_shapes_f16_f32(m, n, k):
    qs = _qs()
    rng = np.random.default_rng(m * 7919 + n * 31 + k)
    w = rng.standard_normal((n, k)).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    wh = w.astype(np.float16)
    say("ragged f", m, n, k)
    y32 = to_host(qs.mul_mat_f32(to_dev(w), to_dev(x)))
    y16 = to_host(qs.mul_mat_f16_f32(to_dev(wh), to_dev(x)))
    assert_close(y32, mul_mat.mul_mat_f32(w, x), TOL_F, "f32")
    assert_close(y16, mul_mat.mul_mat_f16_f32(wh, x), TOL_F, "f16")
    for v in (1, 2, 3):
        y, _ = qs.debug_mul_mat(qs.MM_TYPE_F16, to_dev(wh), to_dev(x), v)
        assert_close(to_host(y), mul_mat.mul_mat_f16_f32(wh, x), TOL_F, f"f16 variant {v}")
    for v in (1, 3):
        y, _ = qs.debug_mul_mat(qs.MM_TYPE_F32, to_dev(w), to_dev(x), v)
        assert_close(to_host(y), mul_mat.mul_mat_f32(w, x), TOL_F, f"f32 variant {v}")


def test_empty_and_zero_k():
    import torch
    qs = _qs()
    say("empty / K=0")
    out = qs.mul_mat_q4_0_f32(torch.zeros((5, 0), dtype=torch.uint8, device="cuda"),
                              torch.zeros((3, 0), dtype=torch.float32, device="cuda"))
    assert out.shape == (3, 5) and bool((out == 0).all())
    out = torch.full((3, 5), 7.0, device="cuda")
    qs.mul_mat_f32(torch.zeros((5, 0), device="cuda"), torch.zeros((3, 0), device="cuda"), out=out)
    assert bool((out == 0).all())
    e = qs.mul_mat_f16_f32(torch.zeros((0, 8), dtype=torch.float16, device="cuda"),
                           torch.zeros((4, 8), device="cuda"))
    assert e.shape == (4, 0)
    e = qs.mul_mat_q4_0_f32(torch.zeros((6, 18), dtype=torch.uint8, device="cuda"),
                            torch.zeros((0, 32), device="cuda"))
    assert e.shape == (0, 6)


def test_zero_blocks_and_extremes():
    # zero rows and blocks, weight scales near the binary16 top, and a src1
    # row whose Q8_0 scales are binary16 subnormals; every kernel family
    # (narrow, wide, and the skinny kernels of 8-, 16- and 32-row passes)
    rng = np.random.default_rng(10)
    n, k = 64, 512
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[3] = 0.0
    w[5, :64] = 0.0
    w[7] *= 1e4
    wq = codec.quantize_q4_0(w)
    for m in (6, 12, 20):
        x = rng.standard_normal((m, k)).astype(np.float32)
        x[1] = 0.0
        x[2, 32:96] = 0.0
        x[4] *= 1e-5
        for v in (1, 2, 3):
            _check_q4_product(to_dev(wq), wq, x, f"zeros/extremes M={m}", v, (0, n))


def test_deterministic_run_to_run():
    import torch
    qs = _qs()
    n, k = 4096, 14336
    wq_dev, _ = _q4_weights(3, 1, n, k)
    for m in (1, 8, 32, 128):
        x = to_dev(workloads.activations(workloads.activation_seed(3, m), m, k))
        say("determinism", m)
        a = qs.mul_mat_q4_0_f32(wq_dev, x)
        b = qs.mul_mat_q4_0_f32(wq_dev, x)
        assert bool(torch.equal(a, b)), m


def test_concurrent_streams_match_serial():
    """Products of every kernel kind issued on two streams at once (each call
    with its own dst and workspace) give the same bits as the same calls run
    one after another: no kernel keeps state outside the caller's buffers."""
    import torch
    qs = _qs()
    n, k = 4096, 4096
    wq_dev, _ = _q4_weights(3, 1, n, k)
    w16 = to_dev(workloads.weights_f16(workloads.weight_seed(2, 0), n, k))
    cases = []
    for m in (1, 2, 8, 40, 512):
        x = to_dev(workloads.activations(workloads.activation_seed(3, m), m, k))
        cases.append((qs.mul_mat_q4_0_f32, wq_dev, x))
    for m in (1, 4, 100):
        x = to_dev(workloads.activations(workloads.activation_seed(2, m), m, k))
        cases.append((qs.mul_mat_f16_f32, w16, x))
    say("concurrent streams", len(cases), "calls")
    serial = [fn(w, x) for fn, w, x in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(y) for y in serial]
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        for i, (fn, w, x) in enumerate(cases):
            with torch.cuda.stream(streams[i % 2]):
                fn(w, x, out=outs[i])
        torch.cuda.synchronize()
        for i, (y, o) in enumerate(zip(serial, outs)):
            assert bool(torch.equal(y, o)), f"call {i} (rep {rep}) differs on its own stream"


def test_graph_capture_replays_match_eager():
    """Every launch sequence the library issues (fused; INIT + skinny; INIT +
    wide + split-K reduce; INIT + wide; F16 pre-pass + wide + reduce; F16
    pre-pass + wide; skinny F16 / F32; narrow F16) captured once into a HIP
    graph and replayed three times, with other products run eagerly on the
    same buffers' neighbours between the replays: every replay gives the
    eager bits."""
    import torch
    qs = _qs()
    rng = np.random.default_rng(5)
    mats = {}

    def weights(kind, n, k):
        key = (kind, n, k)
        if key not in mats:
            w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
            mats[key] = (qs.quantize_q4_0(to_dev(w)) if kind == "q4_0"
                         else to_dev(w.astype(np.float16)) if kind == "f16" else to_dev(w))
        return mats[key]

    shapes = [("q4_0", 1, 4096, 4096), ("q4_0", 8, 4096, 14336), ("q4_0", 128, 4096, 14336),
              ("q4_0", 512, 14336, 4096), ("f16", 100, 4096, 14336), ("f16", 64, 14336, 4096),
              ("f16", 4, 4096, 4096), ("f32", 16, 4096, 4096), ("f16", 1, 4096, 4096)]
    fns = {"q4_0": (qs.mul_mat_q4_0_f32, qs.MM_TYPE_Q4_0), "f16": (qs.mul_mat_f16_f32, qs.MM_TYPE_F16),
           "f32": (qs.mul_mat_f32, qs.MM_TYPE_F32)}
    calls = []
    for kind, m, n, k in shapes:
        fn, t = fns[kind]
        x = to_dev(rng.standard_normal((m, k)).astype(np.float32))
        out = torch.empty((m, n), device="cuda")
        ws = torch.empty(max(qs.workspace_size(t, m, n, k), 1), dtype=torch.uint8, device="cuda")
        calls.append((fn, weights(kind, n, k), x, out, ws, f"{kind} M={m} {n}x{k} {qs.dispatch(t, m, n, k)}"))
    say("graph capture", len(calls), "calls")
    eager = []
    for fn, w, x, out, ws, what in calls:
        fn(w, x, out=out, ws=ws)
        eager.append(out.clone())
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for fn, w, x, out, ws, what in calls:
            fn(w, x, out=out, ws=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        for _, _, _, out, ws, _ in calls:
            out.fill_(float("nan"))
            ws.fill_(0xA5)
        # other eager products between the replays
        for fn, w, x, _, _, _ in calls[:3]:
            fn(w, x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (_, _, _, out, _, what), ref in zip(calls, eager):
            assert bool(torch.equal(out, ref)), f"replay {rep}: {what}"


def test_batch_vs_alone():
    """Row m of a batched product equals the M=1 product of that row (within
    tolerance across kernels; the Q8_0 wdata of the row is identical)."""
    qs = _qs()
    n, k = 14336, 4096
    wq_dev, wq = _q4_weights(3, 0, n, k)
    x = workloads.activations(workloads.activation_seed(3, 64), 64, k)
    say("batch vs alone")
    full = to_host(qs.mul_mat_q4_0_f32(wq_dev, to_dev(x)))
    for i in (0, 17, 63):
        alone = to_host(qs.mul_mat_q4_0_f32(wq_dev, to_dev(x[i:i + 1])))
        assert_close(full[i:i + 1], alone.astype(np.float64), TOL_Q4_0, f"row {i}")


def test_workspace_errors_launch_nothing():
    import torch
    qs = _qs()
    w = torch.zeros((64, 18 * 8), dtype=torch.uint8, device="cuda")
    x = torch.zeros((4, 256), device="cuda")
    out = torch.full((4, 64), 3.0, device="cuda")
    need = qs.workspace_size(qs.MM_TYPE_Q4_0, 4, 64, 256)
    ws = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    st = qs.lib.mm_mul_mat_q4_0_f32(w.data_ptr(), x.data_ptr(), out.data_ptr(), 4, 64, 256,
                                    ws.data_ptr(), need - 1, None)
    assert st == -4
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())


def test_init_compute_stages_equal_the_fused_call():
    """mm_q4_0_init + mm_q4_0_compute gives the same bits as mm_mul_mat_q4_0_f32, and one
    init serves several weight matrices of the same shape (split-K tickets included)."""
    import torch
    qs = _qs()
    for (n, k, m) in ((4096, 4096, 1), (64, 14336, 1), (64, 14336, 32), (4096, 14336, 16)):
        rng = np.random.default_rng(n + k + m)
        x = to_dev(rng.standard_normal((m, k)).astype(np.float32))
        say("init/compute", n, k, m)
        ws = qs.q4_0_init(x, n)
        for rep in range(3):
            w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
            wq = codec.quantize_q4_0(w)
            wq_dev = to_dev(wq)
            y_stage = qs.q4_0_compute(wq_dev, ws, m, k)
            y_fused = qs.mul_mat_q4_0_f32(wq_dev, x)
            assert bool(torch.equal(y_stage, y_fused)), (n, k, m, rep)
            assert_close(to_host(y_stage), mul_mat.mul_mat_q4_0_f32_dequant(wq, to_host(x)),
                         TOL_Q4_0, "staged")


@pytest.mark.parametrize("m", [1, 2, 5, 16, 40])
def test_grouped_products(m):
    """Several products sharing src1 in one grouped call equal the separate calls."""
    import torch
    qs = _qs()
    k = 4096
    rng = np.random.default_rng(70 + m)
    ns = [4096, 1000, 0, 4096, 37]
    ws, wqs = [], []
    for n in ns:
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        wq = codec.quantize_q4_0(w)
        wqs.append(wq)
        ws.append(to_dev(wq) if n else torch.zeros((0, k // 32 * 18), dtype=torch.uint8, device="cuda"))
    x = rng.standard_normal((m, k)).astype(np.float32)
    say("grouped", m, ns)
    outs = qs.mul_mat_q4_0_f32_group(ws, to_dev(x))
    for n, wq, w, out in zip(ns, wqs, ws, outs):
        assert out.shape == (m, n)
        if n == 0:
            continue
        single = qs.mul_mat_q4_0_f32(w, to_dev(x))
        # a member takes the group's kernel (planned for the rows of all
        # members); where the matrix alone is planned the same (same kernel,
        # no split), the same bits
        same = qs.dispatch(qs.MM_TYPE_Q4_0, m, n, k)[:2] == (qs.dispatch(qs.MM_TYPE_Q4_0, m, sum(ns), k)[0], 1)
        if n >= 4096 and same:
            assert bool(torch.equal(out, single))
        assert_close(to_host(out), mul_mat.mul_mat_q4_0_f32_dequant(wq, x), TOL_Q4_0, f"group n={n}")


# Groups of one to three matrices: the fused M <= 2 kernel takes their
# weight pointers and first rows as kernel arguments (row boundaries off the
# workgroup's row groups, a ragged member, the decode step's q,k,v and
# gate,up shapes); larger groups read a descriptor (test_grouped_products).
@pytest.mark.parametrize("m", [1, 2])
@pytest.mark.parametrize("ns", [[4096, 4096, 4096], [1000, 37, 2048], [11008, 11008], [300]])
def test_grouped_products_up_to_three(m, ns):
    import torch
    qs = _qs()
    k = 4096
    rng = np.random.default_rng(90 + m + len(ns) + ns[0])
    ws, wqs = [], []
    for n in ns:
        wq = codec.quantize_q4_0((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
        wqs.append(wq)
        ws.append(to_dev(wq))
    x = rng.standard_normal((m, k)).astype(np.float32)
    say("grouped<=3", m, ns, qs.dispatch(qs.MM_TYPE_Q4_0, m, sum(ns), k))
    outs = qs.mul_mat_q4_0_f32_group(ws, to_dev(x))
    for n, wq, w, out in zip(ns, wqs, ws, outs):
        assert out.shape == (m, n)
        ref = mul_mat.mul_mat_q4_0_f32_dequant(wq, x)
        assert_close(to_host(out), ref, TOL_Q4_0, f"group n={n}")
        # every output of the member equals the matrix computed alone (each
        # wave reduces one weight row in the same order either way)
        single = qs.mul_mat_q4_0_f32(w, to_dev(x))
        same = qs.dispatch(qs.MM_TYPE_Q4_0, m, n, k)[:2] == (qs.dispatch(qs.MM_TYPE_Q4_0, m, sum(ns), k)[0], 1)
        if same:
            assert bool(torch.equal(out, single)), f"group n={n} differs from the single call"


# ------------------------------------------------------- F16 src1 range
# Row scales from far below binary16's normal range to far above its largest
# value, in one batch; an all-zero row among them.  Every F16 path (narrow,
# skinny MFMA in one or several 16-row passes, wide MFMA) must stay within
# the F16 bound on every row, as F32 does.
ROW_SCALES = [1e-30, 1e-7, 1e-5, 1e-3, 1.0, 1e3, 1e5, 0.0, 1e30]


def _scaled_rows(m, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32)
    scales = np.array([ROW_SCALES[i % len(ROW_SCALES)] for i in range(m)], dtype=np.float32)
    return (x * scales[:, None]).astype(np.float32)


@pytest.mark.parametrize("m,n,k", [
    (2, 8200, 4096), (2, 4096, 4096), (4, 4096, 4096), (16, 4096, 4096), (17, 4096, 4096),
    (17, 9000, 1024), (64, 4096, 1024), (64, 8500, 512), (512, 640, 512), (5, 300, 1000),
])
def test_f16_src1_row_scales(m, n, k):
    qs = _qs()
    rng = np.random.default_rng(m * 31 + n + k)
    wh = (rng.standard_normal((n, k)) * 0.02).astype(np.float16)
    x = _scaled_rows(m, k, 1000 + m)
    kind = qs.dispatch(qs.MM_TYPE_F16, m, n, k)[0]
    say("f16 row scales", m, n, k, "variant", kind)
    y = to_host(qs.mul_mat_f16_f32(to_dev(wh), to_dev(x)))
    assert_close(y, mul_mat.mul_mat_f16_f32(wh, x), TOL_F, f"f16 scaled rows {m}x{n}x{k}")
    for v in (1, 2, 3):
        yv, _ = qs.debug_mul_mat(qs.MM_TYPE_F16, to_dev(wh), to_dev(x), v)
        assert_close(to_host(yv), mul_mat.mul_mat_f16_f32(wh, x), TOL_F, f"f16 scaled rows variant {v}")
    w = wh.astype(np.float32)
    y32 = to_host(qs.mul_mat_f32(to_dev(w), to_dev(x)))
    assert_close(y32, mul_mat.mul_mat_f32(w, x), TOL_F, f"f32 scaled rows {m}x{n}x{k}")


@pytest.mark.parametrize("m,n", [(16, 4096), (40, 4096), (100, 11008)])
def test_f16_batch_vs_alone(m, n):
    """Row i of a batched F16 product equals the M = 1 product of that row
    (smallbard 'La courbe': a sequence gives in a batch what it gives alone),
    for rows of very different magnitudes."""
    qs = _qs()
    k = 4096
    rng = np.random.default_rng(m + n)
    wh = (rng.standard_normal((n, k)) * 0.02).astype(np.float16)
    x = _scaled_rows(m, k, 77 + m)
    say("f16 batch vs alone", m, n)
    full = to_host(qs.mul_mat_f16_f32(to_dev(wh), to_dev(x)))
    for i in range(0, m, max(1, m // 12)):
        if not np.any(x[i]):
            continue
        alone = to_host(qs.mul_mat_f16_f32(to_dev(wh), to_dev(x[i:i + 1])))
        assert_close(full[i:i + 1], alone.astype(np.float64), TOL_F, f"row {i}")


@pytest.mark.parametrize("n", [4096, 8192, 8191])
def test_f16_m2_aligned(n):
    """F16 at M = 2 with aligned operands and K % 8 == 0: the dispatched
    (skinny MFMA) kernel and the vectorised narrow kernel (variant 1)."""
    qs = _qs()
    k = 4096
    rng = np.random.default_rng(n)
    wh = (rng.standard_normal((n, k)) * 0.02).astype(np.float16)
    x = rng.standard_normal((2, k)).astype(np.float32)
    say("f16 M=2", n, k, qs.dispatch(qs.MM_TYPE_F16, 2, n, k))
    y = to_host(qs.mul_mat_f16_f32(to_dev(wh), to_dev(x)))
    assert_close(y, mul_mat.mul_mat_f16_f32(wh, x), TOL_F, f"f16 M=2 N={n}")
    y1, _ = qs.debug_mul_mat(qs.MM_TYPE_F16, to_dev(wh), to_dev(x), 1)
    assert_close(to_host(y1), mul_mat.mul_mat_f16_f32(wh, x), TOL_F, f"f16 M=2 N={n} narrow")


@pytest.mark.parametrize("m", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("n,k", [(100, 4096), (300, 2056), (1000, 1032), (8191, 4096), (100, 1001)])
def test_f_narrow_k_slices(m, n, k):
    """The narrow F16 / F32 kernel (variant 1) with its waves splitting K
    over the same rows: two or four slices, uneven and empty last slices
    (K / 8 = 257, 129), clamped rows past N, and K % 8 != 0 (one slice, the
    scalar path) against the oracle."""
    qs = _qs()
    rng = np.random.default_rng(m * 104729 + n * 13 + k)
    w = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    wh = w.astype(np.float16)
    say("f narrow k slices", m, n, k)
    y, _ = qs.debug_mul_mat(qs.MM_TYPE_F16, to_dev(wh), to_dev(x), 1)
    assert_close(to_host(y), mul_mat.mul_mat_f16_f32(wh, x), TOL_F, f"f16 narrow {m}x{n}x{k}")
    y, _ = qs.debug_mul_mat(qs.MM_TYPE_F32, to_dev(w), to_dev(x), 1)
    assert_close(to_host(y), mul_mat.mul_mat_f32(w, x), TOL_F, f"f32 narrow {m}x{n}x{k}")


def test_env_overrides_products():
    """Products planned under MM_NARROW_MAX_M and MM_SPLIT_K (a child
    process: the library reads them once) against the oracle: the narrow
    kernel at M = 5 with its K split 4 ways, the wide kernel split 4 ways."""
    import json
    import os
    import subprocess
    import sys
    import tempfile
    cases = [(5, 300, 16384), (128, 256, 2048)]
    rng = np.random.default_rng(99)
    with tempfile.TemporaryDirectory() as d:
        ins = []
        for i, (m, n, k) in enumerate(cases):
            wq = codec.quantize_q4_0((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
            x = rng.standard_normal((m, k)).astype(np.float32)
            np.save(os.path.join(d, f"w{i}.npy"), wq)
            np.save(os.path.join(d, f"x{i}.npy"), x)
            ins.append((wq, x))
        code = ("import json, os, sys, numpy as np, torch\n"
                "import quantized_skinny_gemm_amd as qs\n"
                "d = sys.argv[1]\n"
                "plans = []\n"
                "for i in range(int(sys.argv[2])):\n"
                "    w = torch.from_numpy(np.load(os.path.join(d, f'w{i}.npy'))).cuda()\n"
                "    x = torch.from_numpy(np.load(os.path.join(d, f'x{i}.npy'))).cuda()\n"
                "    y = qs.mul_mat_q4_0_f32(w, x)\n"
                "    np.save(os.path.join(d, f'y{i}.npy'), y.cpu().numpy())\n"
                "    plans.append(list(qs.dispatch(qs.MM_TYPE_Q4_0, x.shape[0], w.shape[0], x.shape[1])))\n"
                "print(json.dumps(plans))\n")
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        env = dict(os.environ, MM_NARROW_MAX_M="8", MM_SPLIT_K="4")
        say("env overrides child")
        r = subprocess.run([sys.executable, "-c", code, d, str(len(cases))], capture_output=True,
                           text=True, env=env, cwd=root, timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        plans = json.loads(r.stdout.strip().splitlines()[-1])
        assert plans[0][:2] == [1, 4] and plans[1][:2] == [2, 4], plans
        for i, (wq, x) in enumerate(ins):
            y = np.load(os.path.join(d, f"y{i}.npy"))
            assert_close(y, mul_mat.mul_mat_q4_0_f32(wq, x), TOL_Q4_0, f"override case {i}")
