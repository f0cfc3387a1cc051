"""CPU checks of bench.py's work accounting (no GPU)."""
from __future__ import annotations

import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "roofline_smallbard.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = float(v)
    return vals


def test_f32_intensity_and_ridge_match_the_page():
    g = _golden()
    assert bench.f32_weight_intensity(1) == g["ops_per_weight_byte_per_row"]
    # the batch where intensity reaches the device ridge
    assert bench.f32_weight_intensity(g["ridge_rows"]) == g["ridge_ops_per_byte"]


def test_step_ops_and_ideal_time_match_the_page():
    g = _golden()
    weights = g["model_bytes"] / 4            # f32 parameters
    # the model's matrices are N x K with N*K = weights; ops scale as 2*M*N*K
    ops = bench.product_ops(int(g["batch"]), int(weights), 1)
    assert ops == pytest.approx(g["step_ops"], rel=0.02)
    assert ops / g["peak_ops_per_s"] == pytest.approx(g["ideal_step_s"], rel=0.02)


def test_q4_0_step_bytes():
    # weights 0.5625 B/value, src1 read 4 B, Q8_0 wdata written + read 2 x 1.0625 B, dst 4 B
    assert bench.q4_step_bytes(1, 4096, 4096) == 4096 * 4096 * 18 / 32 + 4 * 4096 + 2 * 34 / 32 * 4096 + 4 * 4096
    assert bench.q4_compute_bytes(1, 4096, 4096) == 4096 * 4096 * 18 / 32 + 34 / 32 * 4096 + 4 * 4096
    # one Llama-7B layer at M=1 streams about 113.7 MB of Q4_0 weights
    layer = sum(bench.q4_step_bytes(1, *bench._shapes()[s]) for s in bench.LAYER_SLOTS)
    assert 113e6 < layer < 114.5e6


def test_multi_gpu_request_exits_with_a_message(capsys, monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "8"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
