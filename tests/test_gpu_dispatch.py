"""GPU parity along the measured dispatch table: at the ends of every M range
the committed table lists (shapes up to 14336 rows), the dispatched kernel is
the one the table names and its output matches the oracle (Q4_0: block dots
of sampled columns bit for bit, dst within 1e-5; F16 / F32 within 1e-3)."""
from __future__ import annotations

import os

import numpy as np
import pytest

from oracle import codec, mul_mat
from tests.gpu_util import TOL_F, TOL_Q4_0, assert_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLE = os.path.join(ROOT, "quantized_skinny_gemm_amd", "dispatch_table.txt")


def _cases():
    out = []
    if not os.path.exists(TABLE):
        return out
    for line in open(TABLE):
        f = line.split("#")[0].split()
        if len(f) != 6:
            continue
        t, n, k, lo, hi, v = f[0], int(f[1]), int(f[2]), int(f[3]), int(f[4]), int(f[5])
        if n > 14336:
            continue
        for m in sorted({lo, min(hi, 512, 2 * lo + 1)}):
            out.append((t, n, k, m, v))
    return out


@pytest.mark.parametrize("t,n,k,m,v", _cases())
def test_table_kernel_against_oracle(t, n, k, m, v):
    import torch
    import quantized_skinny_gemm_amd as qs
    mm_type = {"q4_0": qs.MM_TYPE_Q4_0, "q4_0r": qs.MM_TYPE_Q4_0R, "f16": qs.MM_TYPE_F16,
               "f32": qs.MM_TYPE_F32}[t]
    assert qs.dispatch(mm_type, m, n, k)[0] == v
    rng = np.random.default_rng(n * 13 + k * 7 + m)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    cols = np.unique(np.concatenate([np.arange(0, 32), np.arange(n - 32, n),
                                     rng.integers(0, n, 96)]))
    say("table", t, n, k, m, v)
    if t in ("q4_0", "q4_0r"):
        wq = codec.quantize_q4_0(w)
        wd = to_dev(wq)
        if t == "q4_0r":
            wd = qs.repack_q4_0(wd, k)
        out = torch.empty((m, n), dtype=torch.float32, device="cuda")
        dots = torch.empty((m, 32, k // 32), dtype=torch.int32, device="cuda")
        wsb = qs.debug_workspace_size(mm_type, m, n, k, 0)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        x_dev = to_dev(x)
        st = qs.lib.mm_debug_mul_mat(mm_type, wd.data_ptr(), x_dev.data_ptr(), out.data_ptr(),
                                     dots.data_ptr(), m, n, k, n - 32, n, 0, ws.data_ptr(), wsb,
                                     torch.cuda.current_stream().cuda_stream)
        assert st == 0, qs.status_string(st)
        y = to_host(out)[:, cols]
        assert_close(y, mul_mat.mul_mat_q4_0_f32_dequant(wq[cols], x), TOL_Q4_0, f"{t} {m}x{n}x{k}")
        want = codec.block_dots(wq[n - 32:n], codec.quantize_q8_0(x), k)
        assert np.array_equal(to_host(dots), want)
    else:
        if t == "f16":
            wh = w.astype(np.float16)
            y = to_host(qs.mul_mat_f16_f32(to_dev(wh), to_dev(x)))[:, cols]
            ref = mul_mat.mul_mat_f16_f32(wh[cols], x)
        else:
            y = to_host(qs.mul_mat_f32(to_dev(w), to_dev(x)))[:, cols]
            ref = mul_mat.mul_mat_f32(w[cols], x)
        assert_close(y, ref, TOL_F, f"{t} {m}x{n}x{k}")
