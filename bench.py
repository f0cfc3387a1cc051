#!/usr/bin/env python3
"""Throughput of the Q4_0 MUL_MAT at Llama-7B decode shapes on one MI355X.

One step = the weight products of one decoded token of a Llama-7B-shaped
model: 32 layers x 7 products at M = 1 (q, k, v, o: 4096x4096; ffn gate,
up: 11008x4096; ffn down: 4096x11008), each the full product (INIT:
quantize the activation row to Q8_0; COMPUTE: the Q4_0 x Q8_0 product).
The products that share an input -- q, k, v and gate, up -- are issued as
one mm_mul_mat_q4_0_f32_group call each, the others as mm_mul_mat_q4_0_f32:
4 launches per layer.  The same step issued as one call per matrix is
timed too and reported beside it.  The 224 weight matrices are distinct device buffers (3.64 GB of
Q4_0), so every step streams the whole model from HBM, as decode does (the
token reads every weight once: smallbard "Generer a plusieurs", opening
section).  Inputs are resident in HBM before timing starts.

Output: one JSON line on stdout.  `value` is whole-step algorithmic HBM
traffic / step time (GB/s); `roofline` reports the product kernel alone
(HIP events around graph replays of its launches); `cpu_baseline` times the
CPU oracle on a bounded sample of the same work.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--only-step] [--copy-calibration BYTES] [--sweep [JSON]]

--only-step skips the one-call-per-matrix comparison (profiling runs use it,
so that every product launch belongs to the grouped step's mix);
--copy-calibration runs a plain device copy of BYTES ten times and exits
(the reference reading for the HBM byte counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q4_0 mul_mat HBM GB/s (M≤16) and TOPS (M≥32), % of MI355X roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
Q4_BYTES_PER_VALUE = 18 / 32   # Q4_0 block: 18 bytes per 32 values
Q8_BYTES_PER_VALUE = 34 / 32   # Q8_0 block: 34 bytes per 32 values
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_q4_fused_llama7b_decode.json")
NARROW_SRC = os.path.join(ROOT, "quantized_skinny_gemm_amd", "csrc", "q4_narrow.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ----------------------------------------------------------- accounting
def q4_step_bytes(m: int, n: int, k: int) -> float:
    """Algorithmic bytes of one mm_mul_mat_q4_0_f32: Q4_0 weights read once, src1 read,
    Q8_0 wdata written then read once, dst written."""
    return Q4_BYTES_PER_VALUE * n * k + 4.0 * m * k + 2.0 * Q8_BYTES_PER_VALUE * m * k + 4.0 * m * n


def q4_fused_bytes(m: int, n: int, k: int) -> float:
    """Algorithmic bytes of the product when INIT is fused into it: the Q8_0 wdata
    stays in on-chip memory, so only weights, src1 and dst touch HBM."""
    return Q4_BYTES_PER_VALUE * n * k + 4.0 * m * k + 4.0 * m * n


def q4_compute_bytes(m: int, n: int, k: int) -> float:
    """Algorithmic bytes of the COMPUTE kernel alone: weights, wdata read, dst written."""
    return Q4_BYTES_PER_VALUE * n * k + Q8_BYTES_PER_VALUE * m * k + 4.0 * m * n


def f32_weight_intensity(m: int) -> float:
    """Operations per byte of f32 weights read for an M-row product: 2*M*N*K / (4*N*K)."""
    return 2.0 * m / 4.0


def product_ops(m: int, n: int, k: int) -> float:
    return 2.0 * m * n * k


# ------------------------------------------------------------ workload
LAYER_SLOTS = [0, 0, 0, 0, 1, 1, 2]     # q k v o gate up down -> distinct shape index


def _shapes():
    import workloads
    return [workloads.LLAMA7B_LAYER[0], workloads.LLAMA7B_LAYER[4], workloads.LLAMA7B_LAYER[6]]


def setup_gpu(layers: int):
    import numpy as np
    import torch

    import quantized_skinny_gemm_amd as qs
    import workloads

    dev = torch.device("cuda:0")
    shapes = _shapes()
    q4_dev = []
    for j, (n, k) in enumerate(shapes):
        w = workloads.weights_f32(workloads.weight_seed(1, j), n, k)
        q4_dev.append(qs.quantize_q4_0(torch.from_numpy(w).to(dev)))
    # one allocation holding every layer's copy of every slot
    sizes = [q4_dev[s].numel() for s in LAYER_SLOTS]
    per_layer = sum(sizes)
    pool = torch.empty(per_layer * layers, dtype=torch.uint8, device=dev)
    weights = []
    off = 0
    for _ in range(layers):
        row = []
        for s, sz in zip(LAYER_SLOTS, sizes):
            v = pool[off:off + sz].view(q4_dev[s].shape)
            v.copy_(q4_dev[s])
            row.append(v)
            off += sz
        weights.append(row)
    xs = {}
    for n, k in shapes:
        if k not in xs:
            xs[k] = torch.from_numpy(workloads.activations(workloads.activation_seed(1, 1), 1, k)).to(dev)
    dsts = [torch.empty((1, shapes[s][0]), dtype=torch.float32, device=dev) for s in LAYER_SLOTS]
    ws_bytes = max(qs.workspace_size(qs.MM_TYPE_Q4_0, 1, n, k) for n, k in shapes)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    return dict(qs=qs, torch=torch, np=np, shapes=shapes, weights=weights, xs=xs, dsts=dsts,
                ws=ws, ws_bytes=ws_bytes, pool_bytes=pool.numel(), pool=pool)


def _group_args(ws_list, outs, ns):
    import ctypes
    count = len(ws_list)
    src = (ctypes.c_void_p * count)(*[w.data_ptr() for w in ws_list])
    dst = (ctypes.c_void_p * count)(*[o.data_ptr() for o in outs])
    narr = (ctypes.c_int64 * count)(*ns)
    return src, dst, narr


def make_calls(st, stream_handle, grouped: bool):
    """Per layer, the list of (kind, fn, args, bytes) of one decode token's products.
    grouped: q, k, v in one grouped call and gate, up in another (they share src1);
    otherwise one mm_mul_mat_q4_0_f32 per matrix.  Every call goes through the C ABI."""
    lib = st["qs"].lib
    ws, wsb = st["ws"].data_ptr(), st["ws_bytes"]
    layers = []
    for row in st["weights"]:
        calls = []
        if grouped:
            for kind, slots in (("qkv", [0, 1, 2]), ("o", [3]), ("gate_up", [4, 5]), ("down", [6])):
                n_k = [st["shapes"][LAYER_SLOTS[sl]] for sl in slots]
                k = n_k[0][1]
                # src1 is read once per launch
                nbytes = sum(q4_fused_bytes(1, n, k) for n, _ in n_k) - 4.0 * k * (len(slots) - 1)
                if len(slots) == 1:
                    sl = slots[0]
                    args = (row[sl].data_ptr(), st["xs"][k].data_ptr(), st["dsts"][sl].data_ptr(),
                            1, n_k[0][0], k, ws, wsb, stream_handle)
                    calls.append((kind, lib.mm_mul_mat_q4_0_f32, args, nbytes))
                else:
                    src, dst, narr = _group_args([row[sl] for sl in slots],
                                                 [st["dsts"][sl] for sl in slots], [n for n, _ in n_k])
                    st.setdefault("_keep", []).append((src, dst, narr))
                    args = (len(slots), src, dst, narr, st["xs"][k].data_ptr(), 1, k, ws, wsb,
                            stream_handle)
                    calls.append((kind, lib.mm_mul_mat_q4_0_f32_group, args, nbytes))
        else:
            for sl, w in enumerate(row):
                n, k = st["shapes"][LAYER_SLOTS[sl]]
                args = (w.data_ptr(), st["xs"][k].data_ptr(), st["dsts"][sl].data_ptr(), 1, n, k,
                        ws, wsb, stream_handle)
                calls.append((f"{n}x{k}", lib.mm_mul_mat_q4_0_f32, args, q4_fused_bytes(1, n, k)))
        layers.append(calls)
    return layers


def run_calls(calls):
    for c in calls:
        rc = c[1](*c[2])
        if rc != 0:
            raise RuntimeError(f"library call failed with status {rc}")


def time_graph(torch, s, calls, reps):
    """Graph of `calls` on stream s; average ms per replay from HIP events on s."""
    with torch.cuda.stream(s):
        run_calls(calls)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run_calls(calls)
    with torch.cuda.stream(s):
        g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
    s.synchronize()
    return e0.elapsed_time(e1) / reps


def measure_kernels(st, layers, reps: int, s):
    """Average duration per launch of each call kind (every M=1 call here is
    one kernel: INIT fused), from HIP events on the launch stream s (the one
    the calls are bound to) around graph replays of that kind's launches over
    all layers."""
    torch = st["torch"]
    kinds = {}
    for calls in layers:
        for c in calls:
            kinds.setdefault(c[0], []).append(c)
    res = []
    for kind, calls in kinds.items():
        ms = time_graph(torch, s, calls, reps)
        res.append(dict(kind=kind, launches_per_step=len(calls), avg_us=ms * 1e3 / len(calls),
                        bytes=calls[0][3]))
    return res


def traffic_from_profile():
    """HBM bytes per launch of the product kernel (the step's launch mix) from the
    committed rocprofv3 PMC summary, or None when absent or taken on a different
    version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
        with open(NARROW_SRC, "rb") as fh:
            src_hash = hashlib.sha256(fh.read()).hexdigest()
        if t.get("kernel_source_sha256") != src_hash:
            return None
        return float(t["bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def copy_calibration(nbytes: int):
    """A plain device-to-device copy of nbytes, ten times: under rocprofv3 --pmc
    its FETCH_SIZE / WRITE_SIZE give the counters' reading for known traffic."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": a.numel() * 4, "copies": 10}), flush=True)


# ------------------------------------------------------------ config sweep
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published (T op/s)
FP16_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 MFMA, published
MALL_DEFEAT_BYTES = 600e6      # distinct weight copies per timing loop (last-level cache)


def sweep_rows():
    """(workload, type, M, N, K) of every product in the five workloads."""
    import workloads
    rows = []
    for w, spec in workloads.WORKLOADS.items():
        for t in spec["types"]:
            for n, k in spec["shapes"]:
                for m in spec["ms"]:
                    rows.append((w, t, m, n, k))
    return rows


def algo_bytes(t: str, m: int, n: int, k: int, fused: bool) -> float:
    if t == "q4_0":
        return q4_fused_bytes(m, n, k) if fused else q4_step_bytes(m, n, k)
    wb = 2 if t == "f16" else 4
    return wb * n * k + 4.0 * m * k + 4.0 * m * n


def run_sweep(reps: int, out_path: str | None):
    """Times every product of the five workloads (one call per product, HIP
    graph of calls over distinct weight copies, HIP events on the launch
    stream) and reports GB/s, TOPS and the fraction of the bounding roofline."""
    import ctypes
    import torch
    import quantized_skinny_gemm_amd as qs

    dev = torch.device("cuda:0")
    s = torch.cuda.Stream()
    gen = torch.Generator(device=dev)
    results = []
    for (w, t, m, n, k) in sweep_rows():
        mm_type = {"q4_0": qs.MM_TYPE_Q4_0, "f16": qs.MM_TYPE_F16, "f32": qs.MM_TYPE_F32}[t]
        gen.manual_seed(1000 * w + n + k)
        wf = torch.randn((n, k), generator=gen, device=dev, dtype=torch.float32) * 0.02
        if t == "q4_0":
            base = qs.quantize_q4_0(wf)
        elif t == "f16":
            base = wf.to(torch.float16)
        else:
            base = wf
        del wf
        nbytes = base.numel() * base.element_size()
        copies = max(1, min(64, int(-(-MALL_DEFEAT_BYTES // nbytes))))
        if nbytes * copies > 6e9:
            copies = max(1, int(6e9 // nbytes))
        ws_list = [base] + [base.clone() for _ in range(copies - 1)]
        x = torch.randn((m, k), generator=gen, device=dev, dtype=torch.float32)
        dst = torch.empty((m, n), dtype=torch.float32, device=dev)
        wsb = qs.workspace_size(mm_type, m, n, k)
        wsp = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        fn = {"q4_0": qs.lib.mm_mul_mat_q4_0_f32, "f16": qs.lib.mm_mul_mat_f16_f32,
              "f32": qs.lib.mm_mul_mat_f32}[t]
        calls = [(t, fn, (wc.data_ptr(), x.data_ptr(), dst.data_ptr(), m, n, k, wsp.data_ptr(),
                          wsb, s.cuda_stream), 0.0) for wc in ws_list]
        ms = time_graph(torch, s, calls, reps)
        us = ms * 1e3 / len(calls)
        d = (ctypes.c_int * 5)()
        qs.lib.mm_dispatch(mm_type, m, n, k, d)
        variant, split, launches = d[0], d[1], d[4]
        fused = t == "q4_0" and variant == 1 and launches == 1
        nb = algo_bytes(t, m, n, k, fused)
        gbs = nb / (us * 1e-6) / 1e9
        tops = product_ops(m, n, k) / (us * 1e-6) / 1e12
        if t == "q4_0" and m >= 32:
            bound, frac, peak = "int8 MFMA", tops / INT8_PEAK_TOPS, INT8_PEAK_TOPS
        elif t == "f16" and m >= 32:
            bound, frac, peak = "fp16 MFMA", tops / FP16_PEAK_TFLOPS, FP16_PEAK_TFLOPS
        else:
            bound, frac, peak = "hbm", gbs / HBM_PEAK_GBS, None
        # against the lower of the compute peak and what 8 TB/s of the
        # algorithmic bytes allows (M = 32 .. 128 are still HBM-capped)
        cap_frac = frac if peak is None else \
            tops / min(peak, HBM_PEAK_GBS * 1e9 * product_ops(m, n, k) / nb / 1e12)
        r = dict(workload=w, type=t, M=m, N=n, K=k, us=round(us, 3), GBs=round(gbs, 1),
                 TOPS=round(tops, 2), bound=bound, frac=round(frac, 4),
                 frac_of_cap=round(cap_frac, 4),
                 kernel=({1: "narrow", 2: "wide i8", 3: "skinny mfma", 4: "wide fp16"} if t == "q4_0"
                         else {1: "narrow", 2: "wide fp16", 3: "skinny mfma"}).get(variant, str(variant)),
                 split=split, launches=launches,
                 copies=copies)
        results.append(r)
        log(f"w{w} {t:5s} M={m:4d} {n:6d}x{k:<6d} {us:9.3f} us {gbs:8.1f} GB/s {tops:8.2f} TOPS "
            f"{bound:9s} {100 * frac:5.1f}%  ({r['kernel']}, split {split}, {launches} launch)")
        del ws_list, base, x, dst, wsp
        torch.cuda.empty_cache()
    if out_path:
        with open(out_path, "w") as fh:
            json.dump(results, fh, indent=1)
    return results


# ------------------------------------------------------------ dispatch table
TABLE_TYPES = {   # type -> (shapes N x K, kernel variants it has)
    "q4_0": ([(256, 512), (4096, 4096), (11008, 4096), (4096, 11008), (14336, 4096),
              (4096, 14336), (128256, 4096)], (1, 2, 3)),
    "q4_0r": ([(4096, 4096), (11008, 4096), (4096, 11008), (14336, 4096), (4096, 14336),
               (128256, 4096)], (2, 3)),
    "f16": ([(4096, 4096), (11008, 4096), (14336, 4096), (128256, 4096)], (1, 2, 3)),
    "f32": ([(4096, 4096), (11008, 4096)], (1, 3)),
}
TABLE_MS = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]
TABLE_MAX_M = 0x7FFFFFFF


def table_ranges(best):
    """[(M_lo, M_hi, variant)] from {measured M: fastest variant}: each
    crossover at the geometric mean of the measured M on either side, the
    last measured choice kept beyond; adjacent equal choices merged."""
    ms = sorted(best)
    out = []
    for i, m in enumerate(ms):
        lo = 1 if i == 0 else out[-1][1] + 1
        hi = TABLE_MAX_M if i + 1 == len(ms) else int((m * ms[i + 1]) ** 0.5)
        if out and out[-1][2] == best[m]:
            out[-1] = (out[-1][0], hi, best[m])
        else:
            out.append((lo, hi, best[m]))
    return out


def tune_table(path: str, reps: int = 5):
    """Times every kernel variant of every type on the workload shapes at M =
    2^n (graph replays over distinct weight copies, as run_sweep) and writes
    the dispatch table the library reads (one line per M range)."""
    import torch
    import quantized_skinny_gemm_amd as qs

    dev = torch.device("cuda:0")
    s = torch.cuda.Stream()
    gen = torch.Generator(device=dev)
    mm_types = {"q4_0": qs.MM_TYPE_Q4_0, "q4_0r": qs.MM_TYPE_Q4_0R, "f16": qs.MM_TYPE_F16,
                "f32": qs.MM_TYPE_F32}
    lines = ["# Kernel choice per shape, measured on one MI355X by", "#   python bench.py --tune-table <file>",
             "# type N K M_lo M_hi variant   (1 narrow, 2 wide, 3 skinny MFMA)"]
    for t, (shapes, variants) in TABLE_TYPES.items():
        mm_type = mm_types[t]
        for n, k in shapes:
            gen.manual_seed(n + 3 * k)
            wf = torch.randn((n, k), generator=gen, device=dev, dtype=torch.float32) * 0.02
            if t == "q4_0":
                base = qs.quantize_q4_0(wf)
            elif t == "q4_0r":
                base = qs.repack_q4_0(qs.quantize_q4_0(wf), k)
            elif t == "f16":
                base = wf.to(torch.float16)
            else:
                base = wf
            del wf
            nbytes = base.numel() * base.element_size()
            copies = max(1, min(32, int(-(-MALL_DEFEAT_BYTES // nbytes))))
            wcopies = [base] + [base.clone() for _ in range(copies - 1)]
            best = {}
            for m in TABLE_MS:
                x = torch.randn((m, k), generator=gen, device=dev, dtype=torch.float32)
                dst = torch.empty((m, n), dtype=torch.float32, device=dev)
                times = {}
                for v in variants:
                    wsb = qs.debug_workspace_size(mm_type, m, n, k, v)
                    wsp = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
                    torch.cuda.synchronize()
                    calls = [(t, qs.lib.mm_debug_mul_mat,
                              (mm_type, wc.data_ptr(), x.data_ptr(), dst.data_ptr(), None, m, n, k,
                               0, 0, v, wsp.data_ptr(), wsb, s.cuda_stream), 0.0) for wc in wcopies]
                    times[v] = time_graph(torch, s, calls, reps) * 1e3 / len(calls)
                    del wsp
                best[m] = min(times, key=times.get)
                log(f"table {t:5s} {n:6d}x{k:<6d} M={m:4d} " +
                    " ".join(f"v{v} {us:9.2f}us" for v, us in times.items()) + f" -> v{best[m]}")
                del x, dst
            for lo, hi, v in table_ranges(best):
                lines.append(f"{t} {n} {k} {lo} {hi} {v}")
            del wcopies, base
            torch.cuda.empty_cache()
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    log(f"wrote {path}")


# ------------------------------------------------------------ cpu leg
def _oracle_layers(budget_s: float):
    """One worker's leg: the CPU oracle (as it stands) on one Llama-7B layer's 7
    products at M = 1, repeated for about budget_s seconds; returns (layers done,
    wall seconds, cpu seconds).  Weights are quantized by the oracle itself,
    outside the timed loop."""
    import workloads
    from oracle import codec, mul_mat

    shapes = _shapes()
    wq = [codec.quantize_q4_0(workloads.weights_f32(workloads.weight_seed(1, j), n, k))
          for j, (n, k) in enumerate(shapes)]
    xs = {k: workloads.activations(workloads.activation_seed(1, 1), 1, k) for _, k in shapes}
    done = 0
    c0 = os.times()
    t0 = time.perf_counter()
    while True:
        for sl in LAYER_SLOTS:
            n, k = shapes[sl]
            mul_mat.mul_mat_q4_0_f32(wq[sl], xs[k])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    wall = time.perf_counter() - t0
    c1 = os.times()
    return done, wall, (c1.user - c0.user) + (c1.system - c0.system)


def _one_thread_env():
    for v in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[v] = "1"


def _pool_worker(budget_s: float):
    _one_thread_env()
    return _oracle_layers(budget_s)


def cpu_baseline(budget_s: float = 8.0, max_workers: int = 16):
    """The CPU oracle timed on the host: one worker (one thread), then one
    worker per host core (at most max_workers, the host share of one GPU),
    each running the same layer loop on its own copy of the inputs.  Returns
    the all-cores figure with the one-core figure inside it."""
    import multiprocessing as mp

    layer_bytes = sum(q4_step_bytes(1, *_shapes()[sl]) for sl in LAYER_SLOTS)
    ctx = mp.get_context("spawn")
    with ctx.Pool(1) as pool:
        done1, wall1, cpu1 = pool.apply(_pool_worker, (budget_s,))
    workers = max(1, min(max_workers, os.cpu_count() or 1))
    with ctx.Pool(workers) as pool:
        res = pool.map(_pool_worker, [budget_s] * workers)
    done = sum(r[0] for r in res)
    wall = max(r[1] for r in res)
    cpu = sum(r[2] for r in res)
    return {"value": layer_bytes * done / wall / 1e9, "unit": "GB/s",
            "cores": max(1, round(cpu / wall)), "kind": "oracle",
            "sample": f"one Llama-7B layer at M=1 (7 Q4_0 products incl. Q8_0 quantize of "
                      f"src1) repeated: {workers} single-threaded workers x {wall:.1f} s "
                      f"({done} layers); host: {os.cpu_count()} cpus",
            "one_core": {"value": layer_bytes * done1 / wall1 / 1e9, "unit": "GB/s",
                         "cores": max(1, round(cpu1 / wall1)),
                         "sample": f"{done1} layers in {wall1:.1f} s on one thread"}}


# ------------------------------------------------------------ read ceiling
BENCH_READ_LIB = os.path.join(ROOT, "bench_read.so")


READ_GRIDS = (768, 1024, 1536, 2048, 3072, 4096)


def read_ceiling(st, reps: int, s, grids=READ_GRIDS):
    """A plain streaming read (bench_read.so, not the library) of the same
    weight buffers in the same launch pattern as the grouped step: per layer
    q,k,v in one launch, o, gate,up in one, down; 128 launches per step as one
    HIP graph, at each grid size in `grids`.  Returns the best whole-step GB/s
    (weight bytes only) with its grid, the average us per launch of each kind
    at that grid, and the step time at every grid."""
    import ctypes
    torch = st["torch"]
    if not os.path.exists(BENCH_READ_LIB):
        return None
    rl = ctypes.CDLL(BENCH_READ_LIB)
    rl.qsg_bench_stream_read.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                         ctypes.POINTER(ctypes.c_int64), ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    rl.qsg_bench_stream_read.restype = ctypes.c_int
    sink = torch.zeros(max(grids), dtype=torch.int32, device="cuda")
    keep = []
    by_grid = {}
    best = None
    for grid in grids:
        kinds = {}
        step = []
        for row in st["weights"]:
            for kind, slots in (("qkv", [0, 1, 2]), ("o", [3]), ("gate_up", [4, 5]), ("down", [6])):
                ptrs = (ctypes.c_void_p * len(slots))(*[row[sl].data_ptr() for sl in slots])
                nb = (ctypes.c_int64 * len(slots))(*[row[sl].numel() for sl in slots])
                keep.append((ptrs, nb))
                c = (kind, rl.qsg_bench_stream_read,
                     (ptrs, nb, len(slots), sink.data_ptr(), grid, s.cuda_stream),
                     float(sum(row[sl].numel() for sl in slots)))
                step.append(c)
                kinds.setdefault(kind, []).append(c)
        ms = time_graph(torch, s, step, reps)
        by_grid[grid] = round(ms, 5)
        if best is None or ms < best[1]:
            best = (grid, ms, kinds, sum(c[3] for c in step))
    grid, ms, kinds, total = best
    per = {k: round(time_graph(torch, s, v, reps) * 1e3 / len(v), 4) for k, v in kinds.items()}
    return {"GBs": round(total / (ms * 1e-3) / 1e9, 1), "ms_per_step": round(ms, 5),
            "per_kind_us": per, "grid": grid, "ms_per_step_by_grid": by_grid,
            "what": "plain 16-byte streaming read of the step's weight buffers, same 128-launch "
                    "graph (bench_read.hip), best grid of those tried"}


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config table (every product of the five workloads)")
    ap.add_argument("--config-reps", type=int, default=5)
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--only-step", action="store_true",
                    help="only the decode step and its per-launch times (for profiler runs: "
                         "no per-matrix variant, read ceiling or config table)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--tune-table", metavar="FILE",
                    help="time every kernel variant at M = 2^n on the workload shapes and write "
                         "the dispatch table the library reads")
    ap.add_argument("--sweep", metavar="JSON", nargs="?", const="",
                    help="time every product of the five workloads instead (table on "
                         "stderr, optional JSON file)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    if args.sweep is not None:
        run_sweep(max(2, args.kernel_reps // 4), args.sweep or None)
        return
    if args.tune_table:
        tune_table(args.tune_table)
        return

    # the CPU leg first, before this process touches the GPU (its workers are
    # separate processes)
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on 1 core and on all cores (about 20 s)")
        cpu = cpu_baseline()

    st = setup_gpu(args.layers)
    torch = st["torch"]
    shapes = st["shapes"]
    log(f"weights resident: {st['pool_bytes'] / 1e9:.3f} GB Q4_0 in {args.layers} layers x 7")

    s = torch.cuda.Stream()
    grouped = make_calls(st, s.cuda_stream, grouped=True)
    single = make_calls(st, s.cuda_stream, grouped=False)
    step_calls = [c for layer in grouped for c in layer]
    with torch.cuda.stream(s):
        run_calls(step_calls)                   # first call initialises the device check
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        run_calls(step_calls)

    with torch.cuda.stream(s):
        for _ in range(args.warmup):
            graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(s):
        for _ in range(args.steps):
            graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # the same products as one call per matrix (7 launches per layer)
    single_ms = None
    if not args.only_step:
        single_ms = time_graph(torch, s, [c for layer in single for c in layer],
                               max(1, args.steps // 4))

    step_bytes = args.layers * sum(q4_step_bytes(1, *shapes[sl]) for sl in LAYER_SLOTS)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"step {ms_per_step:.4f} ms grouped ({len(step_calls)} launches); {value:.1f} GB/s")
    if single_ms is not None:
        log(f"step {single_ms:.4f} ms as one call per matrix ({len(step_calls) * 7 // 4} launches)")

    kern = measure_kernels(st, grouped, args.kernel_reps, s)
    if not args.only_step:
        for r in measure_kernels(st, single, args.kernel_reps, s):
            log(f"one call per matrix, kernel {r['kind']}: {r['avg_us']:.3f} us/launch, "
                f"{r['bytes'] / (r['avg_us'] * 1e-6) / 1e9:.1f} GB/s")
    tot_bytes = sum(r["bytes"] * r["launches_per_step"] for r in kern)
    tot_us = sum(r["avg_us"] * r["launches_per_step"] for r in kern)
    launches = sum(r["launches_per_step"] for r in kern)
    achieved = tot_bytes / (tot_us * 1e-6) / 1e9
    for r in kern:
        log(f"kernel {r['kind']}: {r['avg_us']:.3f} us/launch, "
            f"{r['bytes'] / (r['avg_us'] * 1e-6) / 1e9:.1f} GB/s")
    traffic = traffic_from_profile()

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "llama7b_decode_q4_0_m1",
            "M": 1,
            "matrices_per_step": args.layers * 7,
            "shapes_NxK": [list(shapes[sl]) for sl in LAYER_SLOTS],
            "layers": args.layers,
            "weights_GB": round(st["pool_bytes"] / 1e9, 4),
            "launch": f"hip graph of {len(step_calls)} calls: per layer q,k,v grouped, o, "
                      "gate,up grouped, down; one kernel each (INIT fused)",
        },
        "tokens_per_s": round(1e3 / ms_per_step, 2),
        "one_call_per_matrix_ms_per_step": None if single_ms is None else round(single_ms, 5),
        "one_call_per_matrix_GBs": None if single_ms is None else
            round(step_bytes / (single_ms * 1e-3) / 1e9, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": "k_q4_fused (INIT fused), M=1, all launches of the step",
            "avg_launch_us": round(tot_us / launches, 4),
            "algorithmic_bytes_per_launch": round(tot_bytes / launches, 1),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "per_kind_us": {r["kind"]: round(r["avg_us"], 4) for r in kern},
        },
    }
    ceiling = None if args.only_step else read_ceiling(st, args.kernel_reps, s)
    if ceiling is not None:
        out["read_ceiling"] = ceiling
        log(f"plain read of the step's weights, same launch pattern: {ceiling['GBs']} GB/s "
            f"({ceiling['per_kind_us']} us per launch)")
    if cpu is not None:
        out["cpu_baseline"] = cpu
    if not args.no_configs and not args.only_step:
        del st, grouped, single, step_calls, graph
        torch.cuda.empty_cache()
        log("timing every product of the five workloads")
        out["configs"] = [
            {k: r[k] for k in ("workload", "type", "M", "N", "K", "us", "GBs", "TOPS", "bound",
                               "frac", "frac_of_cap", "kernel", "launches")}
            for r in run_sweep(args.config_reps, None)]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
