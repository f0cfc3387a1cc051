"""mm_mul_mat_q4_0_f32_noalloc against mm_mul_mat_q4_0_f32, through the C ABI.

The no-allocation entry point runs the same kernels on a fixed device array
instead of a caller workspace, so its output must equal the workspace entry
point's bit for bit (and the oracle within the Q4_0 bound).  Several calls in
a row share the array: each later call is smaller than the one before, so a
stale byte left by an earlier call would show.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import codec, mul_mat
from tests.gpu_util import TOL_Q4_0, assert_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _call_noalloc(qs, wq_dev, x_dev, out):
    import torch
    m, k = x_dev.shape
    n = wq_dev.shape[0]
    st = qs.lib.mm_mul_mat_q4_0_f32_noalloc(wq_dev.data_ptr(), x_dev.data_ptr(), out.data_ptr(),
                                            m, n, k, torch.cuda.current_stream().cuda_stream)
    assert st == 0, qs.status_string(st)
    return out


# (M, N, K): the wide kernel with split-K partials (34.5 MiB of workspace),
# then the skinny MFMA kernel (operand-order wdata), then the fused M = 1
# kernel, each smaller than the one before.
CASES = [(512, 4096, 4096), (8, 1000, 1024), (1, 300, 512)]


def test_noalloc_equals_workspace_entry_point():
    import torch
    import quantized_skinny_gemm_amd as qs
    for i, (m, n, k) in enumerate(CASES):
        rng = np.random.default_rng(4242 + i)
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        x = rng.standard_normal((m, k)).astype(np.float32)
        wq = codec.quantize_q4_0(w)
        wq_dev, x_dev = to_dev(wq), to_dev(x)
        say("noalloc", i, m, n, k, qs.dispatch(qs.MM_TYPE_Q4_0, m, n, k))
        assert qs.workspace_size(qs.MM_TYPE_Q4_0, m, n, k) <= 64 << 20
        want = qs.mul_mat_q4_0_f32(wq_dev, x_dev)
        got = _call_noalloc(qs, wq_dev, x_dev, torch.full((m, n), float("nan"), device="cuda"))
        assert bool(torch.equal(got, want)), f"call {i}: noalloc output differs from the workspace call"
        ref = mul_mat.mul_mat_q4_0_f32_dequant(wq, x)
        assert_close(to_host(got), ref, TOL_Q4_0, f"noalloc call {i}")


def test_noalloc_calls_replayed_from_a_hip_graph():
    """The callers this entry point is for capture it: calls captured into a
    HIP graph (the wide kernel with split-K partials and the skinny kernel
    with its operand-order wdata, both in the shared array) replayed three
    times, with eager no-allocation calls of other shapes rewriting the array
    between the replays, give the workspace entry point's bits every time."""
    import torch
    import quantized_skinny_gemm_amd as qs
    rng = np.random.default_rng(977)
    cap = []
    for m, n, k in ((128, 4096, 14336), (8, 2000, 2048)):
        wq = codec.quantize_q4_0((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
        x_dev = to_dev(rng.standard_normal((m, k)).astype(np.float32))
        wq_dev = to_dev(wq)
        want = qs.mul_mat_q4_0_f32(wq_dev, x_dev)
        cap.append((wq_dev, x_dev, torch.empty((m, n), device="cuda"), want,
                    f"M={m} {n}x{k} {qs.dispatch(qs.MM_TYPE_Q4_0, m, n, k)}"))
    others = []
    for m, n, k in ((512, 4096, 4096), (16, 3000, 1024)):
        wq_dev = to_dev(codec.quantize_q4_0((rng.standard_normal((n, k)) * 0.02).astype(np.float32)))
        others.append((wq_dev, to_dev(rng.standard_normal((m, k)).astype(np.float32)),
                       torch.empty((m, n), device="cuda")))
    say("noalloc graph", [c[4] for c in cap])
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for wq_dev, x_dev, out, _, _ in cap:
            _call_noalloc(qs, wq_dev, x_dev, out)
    torch.cuda.synchronize()
    for rep in range(3):
        for _, _, out, _, _ in cap:
            out.fill_(float("nan"))
        for wq_dev, x_dev, out in others:
            _call_noalloc(qs, wq_dev, x_dev, out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for _, _, out, want, what in cap:
            assert bool(torch.equal(out, want)), f"replay {rep}: {what}"


def test_noalloc_rejects_oversize_shape_and_launches_nothing():
    import torch
    import quantized_skinny_gemm_amd as qs
    m, n, k = 4096, 64, 16384          # wdata alone is 64 MiB + scales
    assert qs.workspace_size(qs.MM_TYPE_Q4_0, m, n, k) > 64 << 20
    out = torch.full((4, 4), 3.0, device="cuda")
    st = qs.lib.mm_mul_mat_q4_0_f32_noalloc(out.data_ptr(), out.data_ptr() + 4096, out.data_ptr(),
                                            m, n, k, None)
    assert st == -4
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
