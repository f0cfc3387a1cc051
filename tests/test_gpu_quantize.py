"""GPU parity of the Q4_0 / Q8_0 quantize kernels against the oracle: bytes must be equal."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import codec
from tests.gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _qs():
    import quantized_skinny_gemm_amd as qs
    return qs


def _check_q4(x: np.ndarray, what: str):
    say("quantize_q4_0", what, x.shape)
    got = to_host(_qs().quantize_q4_0(to_dev(x)))
    want = codec.quantize_q4_0(x)
    bad = np.nonzero(np.any(got != want, axis=1))[0]
    assert bad.size == 0, f"{what}: {bad.size} rows differ, first {bad[:5]}"


def _check_q8(x: np.ndarray, what: str):
    say("quantize_q8_0", what, x.shape)
    got = to_host(_qs().quantize_q8_0(to_dev(x)))
    want = codec.quantize_q8_0(x)
    bad = np.nonzero(np.any(got != want, axis=1))[0]
    assert bad.size == 0, f"{what}: {bad.size} rows differ, first {bad[:5]}"


@pytest.mark.parametrize("wl", [0, 1, 3])
def test_q4_0_weights_of_workloads(wl):
    cfg = workloads.WORKLOADS[wl]
    for j, (n, k) in enumerate(cfg["shapes"]):
        _check_q4(workloads.weights_f32(workloads.weight_seed(wl, j), n, k), f"wl{wl} w{j}")


def test_q4_0_weights_of_prefill_workload_sampled_rows():
    """The 128256 x 4096 projection: all rows quantized on the GPU, sampled rows checked."""
    qs = _qs()
    import torch
    cfg = workloads.WORKLOADS[4]
    for j, (n, k) in enumerate(cfg["shapes"]):
        seed = workloads.weight_seed(4, j)
        w = workloads.weights_f32(seed, n, k)
        say("quantize_q4_0 prefill", j, w.shape)
        got = qs.quantize_q4_0(to_dev(w))
        rows = np.unique(np.concatenate([
            np.arange(0, 64), np.arange(n - 64, n),
            np.random.default_rng(7 + j).integers(0, n, 2048)]))
        sel = to_host(got[torch.from_numpy(rows).cuda()])
        want = codec.quantize_q4_0(workloads.weights_f32(seed, n, k, rows=rows))
        assert np.array_equal(sel, want)
        del got
        torch.cuda.empty_cache()


@pytest.mark.parametrize("wl", [0, 1, 2, 3, 4])
def test_q8_0_activations_of_workloads(wl):
    cfg = workloads.WORKLOADS[wl]
    ks = sorted({k for _, k in cfg["shapes"]})
    for m in cfg["ms"]:
        for k in ks:
            _check_q8(workloads.activations(workloads.activation_seed(wl, m), m, k), f"wl{wl} M={m} K={k}")


def test_hand_worked_golden_blocks():
    from tests.test_oracle_codec import GOLDEN_CASES
    qs = _qs()
    for case in GOLDEN_CASES:
        x = case["x"].reshape(1, 32)
        say("golden", case["name"])
        fn = qs.quantize_q4_0 if case["type"] == "q4_0" else qs.quantize_q8_0
        got = to_host(fn(to_dev(x)))
        assert got.tobytes() == case["bytes"], case["name"]


def test_edge_blocks():
    """Zero blocks, signed-absmax ties, tiny (fp16-subnormal scale) and huge blocks,
    exact code boundaries, and values a few ulps either side of them."""
    rng = np.random.default_rng(5)
    rows = []
    rows.append(np.zeros(64, dtype=np.float32))
    rows.append(np.full(64, -0.0, dtype=np.float32))
    t = np.zeros(64, dtype=np.float32)
    t[0], t[1], t[33], t[40] = -3, 3, 5, -5
    rows.append(t)
    rows.append((rng.standard_normal(64) * 1e-6).astype(np.float32))     # fp16-subnormal d
    rows.append((rng.standard_normal(64) * 3e4).astype(np.float32))
    b = np.zeros(64, dtype=np.float32)
    b[0] = -8.0
    b[1:32] = ((np.arange(31) % 15) - 7.5).astype(np.float32)            # t = x/d + 8.5 integral
    b[32] = 127
    b[33:] = (np.arange(31) - 15.5).astype(np.float32)                   # Q8_0 ties at d = 1
    rows.append(b)
    # a few ulps around Q4_0 code boundaries
    mx = np.float32(-1.7)
    d = mx / np.float32(-8)
    c = np.zeros(64, dtype=np.float32)
    c[0] = mx
    base = (np.arange(1, 32) % 15 + 1 - 8.5).astype(np.float32) * d
    for s in (-2, -1, 1, 2):
        cc = c.copy()
        cc[1:32] = base
        for _ in range(abs(s)):
            cc[1:32] = np.nextafter(cc[1:32], np.float32(np.sign(s) * np.inf), dtype=np.float32)
        cc[32:] = cc[:32]
        rows.append(cc)
    x = np.stack(rows).astype(np.float32)
    _check_q4(x, "edge")
    _check_q8(x, "edge")


def test_random_shapes_and_scales():
    rng = np.random.default_rng(6)
    for rows, k in ((1, 32), (3, 96), (17, 1056), (257, 4128)):
        x = (rng.standard_normal((rows, k)) * rng.choice([1e-3, 0.02, 1.0, 50.0])).astype(np.float32)
        _check_q4(x, f"{rows}x{k}")
        _check_q8(x, f"{rows}x{k}")


def test_batch_invariance_of_wdata():
    """Row m of the Q8_0 wdata is byte-identical whatever M it was quantized in."""
    x = workloads.activations(workloads.activation_seed(3, 128), 128, 4096)
    qs = _qs()
    full = to_host(qs.quantize_q8_0(to_dev(x)))
    for lo, hi in ((0, 1), (5, 13), (100, 128)):
        part = to_host(qs.quantize_q8_0(to_dev(x[lo:hi])))
        assert np.array_equal(part, full[lo:hi])
