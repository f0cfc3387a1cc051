"""GPU parity of the repacked Q4_0 weights (mm_repack_q4_0, mm_unpack_q4_0,
mm_mul_mat_q4_0r_f32).

The repacked layout is a permutation of the Q4_0 bytes plus padding; it is
restated here on the CPU from its definition (include/mm.h) and the GPU
repack must produce the same bytes, unpack must restore the original bytes,
and the product on repacked weights must give the oracle's int32 block dots
bit for bit and dst within the Q4_0 bound, on every kernel it dispatches to.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import codec, mul_mat
from tests.gpu_util import TOL_Q4_0, assert_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu

CHUNK = 2304


def _qs():
    import quantized_skinny_gemm_amd as qs
    return qs


def repack_reference(wq: np.ndarray, n: int, k: int) -> np.ndarray:
    """The repacked layout written out: per 16-row tile and phase of 8
    blocks, codes [half][lane i + 16 g][4 blocks] as code bytes 4g..4g+3 of
    row i, then scales [row][block]; padding codes 0x88, scale 0."""
    nb = k // 32
    tiles, phases = -(-n // 16), -(-nb // 8)
    blocks = np.full((tiles * 16, phases * 8, 18), 0, dtype=np.uint8)
    blocks[:, :, 2:] = 0x88
    blocks[:n, :nb] = wq.reshape(n, nb, 18)
    out = np.empty((tiles, phases, CHUNK), dtype=np.uint8)
    for t in range(tiles):
        for f in range(phases):
            c = out[t, f]
            for b in range(8):
                hh, j = divmod(b, 4)
                for i in range(16):
                    blk = blocks[16 * t + i, 8 * f + b]
                    for g in range(4):
                        off = hh * 1024 + (i + 16 * g) * 16 + 4 * j
                        c[off:off + 4] = blk[2 + 4 * g: 6 + 4 * g]
                    c[2048 + 16 * i + 2 * b: 2048 + 16 * i + 2 * b + 2] = blk[0:2]
    return out.reshape(-1)


@pytest.mark.parametrize("n,k", [(16, 256), (37, 544), (100, 4096), (5, 32)])
def test_repack_bytes_and_round_trip(n, k):
    qs = _qs()
    rng = np.random.default_rng(n * 131 + k)
    wq = codec.quantize_q4_0((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    say("repack", n, k)
    assert qs.repacked_bytes(n, k) == -(-n // 16) * -(-(k // 32) // 8) * CHUNK
    wr = qs.repack_q4_0(to_dev(wq), k)
    assert np.array_equal(to_host(wr), repack_reference(wq, n, k))
    back = qs.unpack_q4_0(wr, n, k)
    assert np.array_equal(to_host(back), wq)


def _debug_r(wr, n, x, variant, n0, n1):
    """mm_debug_mul_mat on repacked weights through the C ABI: dst and the
    int32 block dots of columns n0..n1-1 written by the production kernel."""
    import torch
    qs = _qs()
    m, k = x.shape
    out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    dots = None
    if n1 > n0:
        dots = torch.empty((m, n1 - n0, k // 32), dtype=torch.int32, device=x.device)
    wsb = qs.debug_workspace_size(qs.MM_TYPE_Q4_0R, m, n, k, variant)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=x.device)
    st = qs.lib.mm_debug_mul_mat(qs.MM_TYPE_Q4_0R, wr.data_ptr(), x.data_ptr(), out.data_ptr(),
                                 None if dots is None else dots.data_ptr(), m, n, k, n0, n1,
                                 variant, ws.data_ptr(), wsb,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == 0, qs.status_string(st)
    return out, dots


def _check_r(wq, x, what, variant=0, cols=None, wr=None):
    """Product on repacked weights against the oracle: dst within the bound,
    block dots of columns cols bit for bit; the production entry point gives
    the same bits as the dispatched debug call."""
    import torch
    qs = _qs()
    m, k = x.shape
    n = wq.shape[0]
    if wr is None:
        wr = qs.repack_q4_0(to_dev(wq), k)
    n0, n1 = cols if cols is not None else (0, n)
    say("q4_0r", what, m, n, k, variant, qs.dispatch(qs.MM_TYPE_Q4_0R, m, n, k))
    x_dev = to_dev(x)
    y, dots = _debug_r(wr, n, x_dev, variant, n0, n1)
    ref = mul_mat.mul_mat_q4_0_f32_dequant(wq, x)
    assert_close(to_host(y), ref, TOL_Q4_0, what)
    if dots is not None:
        want = codec.block_dots(wq[n0:n1], codec.quantize_q8_0(x), k)
        assert np.array_equal(to_host(dots), want), f"{what}: block dots differ"
    if variant == 0:
        y2 = qs.mul_mat_q4_0r_f32(wr, n, x_dev)
        assert bool(torch.equal(y, y2)), f"{what}: production call differs from the dump call"
    return to_host(y)


# M = 1 .. 512 through the skinny (M <= 32) and wide kernels; ragged N and K
# (tiles and phases with padding, K off the 256-value phase).
@pytest.mark.parametrize("m,n,k", [
    (1, 300, 512), (2, 100, 1056), (5, 17, 64), (8, 129, 2080), (16, 64, 4096), (17, 250, 800),
    (32, 48, 128), (33, 65, 3200), (64, 200, 1024), (130, 33, 8192), (512, 70, 256),
])
def test_repacked_products_ragged(m, n, k):
    qs = _qs()
    rng = np.random.default_rng(m * 7_000_001 + n * 31 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    wq = codec.quantize_q4_0(w)
    wr = qs.repack_q4_0(to_dev(wq), k)
    cols = (0, min(n, 40))
    _check_r(wq, x, f"ragged {m}x{n}x{k}", 0, cols, wr)
    _check_r(wq, x, f"ragged {m}x{n}x{k} skinny", 3, cols, wr)
    _check_r(wq, x, f"ragged {m}x{n}x{k} wide", 2, cols, wr)


@pytest.mark.parametrize("j", [0, 1])
def test_repacked_llama3_ffn_batched(j):
    """The batched-decode workload on repacked weights: M = 8 .. 128."""
    qs = _qs()
    n, k = workloads.WORKLOADS[3]["shapes"][j]
    w = workloads.weights_f32(workloads.weight_seed(3, j), n, k)
    wq = codec.quantize_q4_0(w)
    wr = qs.repack_q4_0(to_dev(wq), k)
    for m in workloads.WORKLOADS[3]["ms"]:
        x = workloads.activations(workloads.activation_seed(3, m), m, k)
        _check_r(wq, x, f"ffn w{j} M={m}", 0, (n - 64, n), wr)


def test_repacked_decode_and_batch_vs_alone():
    """M = 1 on repacked weights (skinny kernel) and row-wise agreement of a
    batch with the rows computed alone, on the 7B decode shape."""
    qs = _qs()
    n, k = 4096, 4096
    w = workloads.weights_f32(workloads.weight_seed(1, 0), n, k)
    wq = codec.quantize_q4_0(w)
    wr = qs.repack_q4_0(to_dev(wq), k)
    x1 = workloads.activations(workloads.activation_seed(1, 1), 1, k)
    _check_r(wq, x1, "7B decode M=1", 0, (0, n), wr)
    x = workloads.activations(workloads.activation_seed(3, 24), 24, k)
    full = to_host(qs.mul_mat_q4_0r_f32(wr, n, to_dev(x)))
    for i in (0, 9, 23):
        alone = to_host(qs.mul_mat_q4_0r_f32(wr, n, to_dev(x[i:i + 1])))
        assert_close(full[i:i + 1], alone.astype(np.float64), TOL_Q4_0, f"row {i}")
