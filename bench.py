#!/usr/bin/env python3
"""One-GPU benchmark of the Mamba-3 SISO forward path on MI355X.

A step is one pass of the whole SISO hot path over one batch of the
B4 L2048 H24 P64 N128 A32 layer: m3_siso_fwd_packed, the preprocess of the
packed projection [8192, 3432] fused into the scan.  The same pass as two
calls (m3_preprocess, then m3_siso_fwd) is timed beside it.  Inputs for
three independent batches are resident in HBM before timing and are rotated
so the 256 MB last-level cache cannot hold a whole step's working set.

Prints one JSON line: tokens/s of the step, the scan kernel's roofline
(algorithmic bytes / live HIP-event duration against 8 TB/s) beside the same
bytes over the whole scan call (summary pass + main pass) and over the whole
step, and the float64 CPU oracle timed on the host cores (all cores, and one
thread).  Before the warmup it measures the other rows of the path at their
own workloads ("rows"), which also brings the GPU to the clocks it holds
under load before the step is timed: the long-sequence scan at
B1 L65536 H32 (dt in [1e-3, 0.01]), the decode step at B256 H32 (1 token per
step, HBM-bound), the rank-4 MIMO decode step at the same geometry, the MIMO
scan at B8 L4096 H32 R4 (FP32-matrix-bound), the SISO backward at the step's
geometry, the MIMO backward at the MIMO scan's geometry and the preprocess
backward over the step's packed projection.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""

from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, GB/s
FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 (vector and matrix)
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_b4_l2048_traffic.json")
MAIN_KERNEL = "scan_chunk_kernel<4, true, false, 8, 4, 8, 1, true>"  # main pass on the packed rows (the step)
DENSE_KERNEL = "scan_chunk_kernel<4, true, false, 8, 4, 8, 1, false>"  # main pass on dense operands
COPY_KERNEL = "neg_kernel"  # torch.neg over a float32 buffer: reads and writes n*4 bytes once


def kernel_source_hash() -> str:
    """sha256 over the sources the scan kernel is compiled from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_mamba3_amd", "csrc")
    for name in ("scan_fwd.hip", "common.h", "launch.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed steps right before the timed ones (the rows, measured first, already "
                         "bring the GPU to its steady clocks)")
    ap.add_argument("--sets", type=int, default=3, help="input sets rotated through the timed loop")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=24, help="heads in the one-thread oracle's timed sample")
    ap.add_argument("--cpu-decode-steps", type=int, default=32,
                    help="decode steps in the decode row's oracle baseline (0: skip the rows' baselines)")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run plain device copies of this many MiB (counter calibration)")
    ap.add_argument("--summarize", nargs=3, metavar=("STATS_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="summarise rocprofv3 kernel-stats / FETCH_SIZE / WRITE_SIZE output into profiles/")
    ap.add_argument("--calib-mib", type=int, default=256, help="copy size used in the calibrated runs")
    ap.add_argument("--no-rows", action="store_true", help="skip the decode-step and MIMO measurements")
    return ap.parse_args()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_pass(hs, heads):
    """The float64 oracle over the step's packed projection: preprocess of
    every row, then the scan of `heads` over every batch row and token.
    Returns (preprocess seconds, scan seconds)."""
    import oracle as O
    from workloads import WORKLOADS
    d = WORKLOADS["siso_b4_l2048"].dims
    B, L, H, G, P, N, A = d.B, d.L, d.H, d.groups, d.P, d.N, d.A
    ocfg = O.PreprocessConfig(H * P, N, H, A, G, 1, 1e-5, 1e-3, 0.1, 1e-4)
    c0 = time.perf_counter()
    pre = O.preprocess(hs["projected"], hs["dt_bias"], ocfg)
    t_pre = time.perf_counter() - c0
    shp = {"x": (B, L, H, P), "z": (B, L, H, P), "bh": (B, L, G, N), "ch": (B, L, G, N),
           "dt": (B, L, H), "adt": (B, L, H), "trap": (B, L, H), "angle": (B, L, A)}
    oi = {k: pre[k].reshape(shp[k]) for k in shp}
    c0 = time.perf_counter()
    O.siso_scan(oi["ch"], oi["bh"], oi["x"], oi["z"], oi["adt"], oi["dt"], oi["trap"], oi["angle"],
                hs["c_bias"], hs["b_bias"], hs["d"], O.SsmConfig(B, L, H, G, P, N, A), heads=list(heads))
    return t_pre, time.perf_counter() - c0


def _oracle_shard(heads):
    """One process of the multi-core baseline: its own copy of the seeded
    packed projection (not timed), the whole preprocess, its heads' scan."""
    from workloads import WORKLOADS, packed_projection
    w = WORKLOADS["siso_b4_l2048"]
    return _oracle_pass(packed_projection(w.dims, seed=w.seed, dt_range=w.dt_range), heads)


def _spawn_pool_map(fn, tasks):
    """map fn over tasks in min(16, cores) spawned processes of one thread each."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    n = max(1, min(16, os.cpu_count() or 1, len(tasks)))
    keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in keys}
    for k in keys:
        os.environ[k] = "1"
    try:
        with ProcessPoolExecutor(n, mp_context=mp.get_context("spawn")) as pool:
            return n, list(pool.map(fn, tasks))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def oracle_all_cores(H: int):
    """The oracle over all H heads sharded across min(16, cores) spawned
    processes (one thread each).  The job's time is its slowest shard:
    every shard repeats the preprocess, which a shared run would split."""
    n = max(1, min(16, os.cpu_count() or 1, H))
    shards = [list(range(H))[i::n] for i in range(n)]
    n, res = _spawn_pool_map(_oracle_shard, shards)
    crit = max(tp + ts for tp, ts in res)
    return n, crit, float(np.median([tp for tp, _ in res])), max(len(s) for s in shards)


def _row_shard(task):
    """One process of a row's oracle baseline: the workload's seeded inputs
    (not timed), then the oracle over this shard's heads (scans) or batch
    rows (decode).  Returns the oracle's own seconds."""
    import oracle as O
    from workloads import WORKLOADS, Dims, decode_states, ssm_inputs, step_inputs
    name, part, steps = task
    w = WORKLOADS[name]
    d = w.dims
    ops = ("c", "b", "x", "z", "adt", "dt", "trap", "angle", "c_bias", "b_bias", "d")
    cfg = O.SsmConfig(d.B, d.L, d.H, d.G, d.P, d.N, d.A, d.R, d.has_z, d.has_d, d.has_output_norm)
    if w.kind in ("siso", "mimo"):
        inp = ssm_inputs(d, seed=w.seed, dt_range=w.dt_range, mimo=w.kind == "mimo")
        c0 = time.perf_counter()
        if w.kind == "mimo":
            O.mimo_scan(*[inp[k] for k in ops + ("mimo_x", "mimo_z", "mimo_o", "norm_weight")], cfg, heads=part)
        else:
            O.siso_scan(*[inp[k] for k in ops], cfg, heads=part)
        return time.perf_counter() - c0
    rows = np.asarray(part)
    keys = ("ssm_state", "angle_state", "k_state", "v_state")
    st = {k: v[rows].astype(np.float64) for k, v in decode_states(d, seed=w.seed).items()}
    sub = O.SsmConfig(len(rows), 1, d.H, d.G, d.P, d.N, d.A)
    t = 0.0
    for s in range(steps):
        tok = {k: (v[rows] if v.ndim >= 3 else v) for k, v in step_inputs(d, w.seed, s).items()}
        c0 = time.perf_counter()
        _, st = O.siso_step(*[tok[k] for k in ops], *[st[k] for k in keys], sub)
        t += time.perf_counter() - c0
    return t


def oracle_rows_all_cores(decode_steps: int):
    """The oracle baselines of the other scan and decode rows, each over all
    host cores: the long-sequence SISO scan and the MIMO scan sharded by head
    (all heads), the decode step sharded by batch row over its first
    `decode_steps` steps.  Each row's time is its slowest process."""
    from workloads import WORKLOADS
    out = {}
    for row, name in (("siso_long_scan", "siso_long_l65536"), ("mimo_scan", "mimo_b8_l4096_r4")):
        d = WORKLOADS[name].dims
        n = max(1, min(16, os.cpu_count() or 1, d.H))
        n, res = _spawn_pool_map(_row_shard, [(name, list(range(d.H))[i::n], 0) for i in range(n)])
        crit = max(res)
        out[row] = {"value": d.B * d.L / crit, "unit": "tokens/s", "cores": n, "kind": "oracle",
                    "sample": f"float64 oracle, all {d.H} heads of {name} sharded over {n} processes; "
                              f"time = slowest process, {crit:.2f} s (input generation not timed)"}
    w = WORKLOADS["decode_b256"]
    d = w.dims
    n = max(1, min(16, os.cpu_count() or 1, d.B))
    n, res = _spawn_pool_map(_row_shard, [("decode_b256", list(range(d.B))[i::n], decode_steps) for i in range(n)])
    crit = max(res)
    out["decode_step"] = {"value": d.B * decode_steps / crit, "unit": "tokens/s", "cores": n, "kind": "oracle",
                          "sample": f"float64 oracle, the first {decode_steps} of the {w.steps} decode_b256 steps "
                                    f"over all {d.B} batch rows sharded over {n} processes; time = slowest "
                                    f"process, {crit:.2f} s (input generation not timed)"}
    return out


def decode_algorithmic_bytes(B, H, G, P, N, A) -> int:
    """State read and written once, the small states read and written, the
    token operands read and out written (fp32)."""
    return 4 * (2 * B * H * P * N + 2 * B * G * N + 3 * B * H * P + 3 * B * H + B * A
                + 2 * B * H * A + 2 * B * H * N + 2 * B * H * P + 2 * H * N + H)


def measure_rows(torch, m3, lib, hip, new_event, dev):
    """Decode-step, MIMO-scan and backward rows, each at its own workload, timed
    with HIP events on the stream the kernels run on."""
    from workloads import WORKLOADS, decode_states, mimo_decode_states, ssm_inputs, step_inputs
    ops11 = ("c", "b", "x", "z", "adt", "dt", "trap", "angle", "c_bias", "b_bias", "d")
    rows = {}
    f = ctypes.c_float()

    # decode: 256 x 32 heads, state [256, 32, 64, 128]; eight staged token sets
    w = WORKLOADS["decode_b256"]
    d = w.dims
    st = {k: torch.from_numpy(v).to(dev) for k, v in decode_states(d, w.seed).items()}
    toks = [{k: torch.from_numpy(v).to(dev) for k, v in step_inputs(d, w.seed, s).items()} for s in range(8)]
    cfg = m3.SsmConfig(d.B, 1, d.H, d.G, d.P, d.N, d.A)
    out = torch.empty(d.B, 1, d.H, d.P, device=dev)

    def one(i):
        t = toks[i % len(toks)]
        m3.m3_siso_step(*[t[k] for k in ops11], st["ssm_state"], st["angle_state"], st["k_state"],
                        st["v_state"], cfg, out=out)
    for i in range(20):
        one(i)
    torch.cuda.synchronize()
    n_steps = 256
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n_steps):
        one(i)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / n_steps
    byt = decode_algorithmic_bytes(d.B, d.H, d.groups, d.P, d.N, d.A)
    rows["decode_step"] = {"workload": "decode_b256: B256 H32 P64 N128 A32, one token per step",
                           "us_per_step": us, "tokens_per_s": d.B / (us * 1e-6),
                           "algorithmic_bytes": byt, "gbs": byt / (us * 1e-6) / 1e9,
                           "hbm_frac": byt / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "bound": "hbm",
                           "steps_timed": n_steps}
    del st, toks, out

    # MIMO decode: 256 x 32 heads, rank 4, output norm; eight staged token sets
    w = WORKLOADS["mimo_decode_b256_r4"]
    d = w.dims
    st = {k: torch.from_numpy(v).to(dev) for k, v in mimo_decode_states(d, w.seed).items()}
    toks = [{k: torch.from_numpy(v).to(dev) for k, v in step_inputs(d, w.seed, s, mimo=True).items()}
            for s in range(8)]
    cfg = m3.SsmConfig(d.B, 1, d.H, d.G, d.P, d.N, d.A, d.R, True, True, True)
    out = torch.empty(d.B, 1, d.H, d.P, device=dev)
    ops15 = ops11 + ("mimo_x", "mimo_z", "mimo_o", "norm_weight")

    def one_m(i):
        t = toks[i % len(toks)]
        m3.m3_mimo_step(*[t[k] for k in ops15], st["ssm_state"], st["angle_state"], st["k_state"],
                        st["v_state"], cfg, out=out)
    for i in range(20):
        one_m(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n_steps):
        one_m(i)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / n_steps
    Bd, Hd, Gd, Pd, Nd, Ad, Rd = d.B, d.H, d.groups, d.P, d.N, d.A, d.R
    byt = 4 * (2 * Bd * Hd * Pd * Nd + 2 * Bd * Rd * Gd * Nd + 3 * Bd * Hd * Pd + 3 * Bd * Hd + Bd * Ad
               + 2 * Bd * Hd * Ad + 2 * Bd * Hd * Rd * Nd + 2 * Bd * Hd * Rd * Pd + 2 * Hd * Rd * Nd + Hd
               + 3 * Hd * Rd * Pd + Hd * Pd)
    rows["mimo_decode_step"] = {"workload": "mimo_decode_b256_r4: B256 H32 P64 N128 A32 R4, output norm, one token per step",
                                "us_per_step": us, "tokens_per_s": Bd / (us * 1e-6),
                                "algorithmic_bytes": byt, "gbs": byt / (us * 1e-6) / 1e9,
                                "hbm_frac": byt / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "bound": "hbm",
                                "steps_timed": n_steps}
    del st, toks, out

    # MIMO: B8 L4096 H32 P64 N128 A32 R4 with output norm
    w = WORKLOADS["mimo_b8_l4096_r4"]
    d = w.dims
    inp = {k: torch.from_numpy(v).to(dev) for k, v in ssm_inputs(d, seed=w.seed, dt_range=w.dt_range).items()}
    cfg = m3.SsmConfig(d.B, d.L, d.H, d.G, d.P, d.N, d.A, d.R, True, True, True)
    ops = [inp[k] for k in ops11 + ("mimo_x", "mimo_z", "mimo_o", "norm_weight")]
    ws = torch.empty(max(1, m3.mimo_fwd_workspace_bytes(cfg)), dtype=torch.uint8, device=dev)
    out = torch.empty(d.B, d.L, d.H, d.P, device=dev)
    for _ in range(3):
        m3.m3_mimo_fwd(*ops, cfg, out=out, workspace=ws)
    torch.cuda.synchronize()
    kms, cms = [], []
    for _ in range(10):
        e0, e1 = new_event(), new_event()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        lib.m3_set_profile_events(e0, e1)
        a.record()
        m3.m3_mimo_fwd(*ops, cfg, out=out, workspace=ws)
        b.record()
        torch.cuda.synchronize()
        lib.m3_set_profile_events(None, None)
        hip.hipEventElapsedTime(ctypes.byref(f), e0, e1)
        kms.append(f.value)
        cms.append(a.elapsed_time(b))
        hip.hipEventDestroy(e0)
        hip.hipEventDestroy(e1)
    km, cm = float(np.median(kms)), float(np.median(cms))
    Bm, Lm, Hm, Gm, Pm, Nm, Am, Rm = d.B, d.L, d.H, d.groups, d.P, d.N, d.A, d.R
    flops = 4 * Rm * Nm * Pm * Bm * Lm * Hm
    byt = 4 * (3 * Bm * Lm * Hm * Pm + 2 * Bm * Lm * Rm * Gm * Nm + 3 * Bm * Lm * Hm + Bm * Lm * Am
               + 2 * Hm * Rm * Nm + Hm + 3 * Hm * Rm * Pm + Hm * Pm)
    rows["mimo_scan"] = {"workload": "mimo_b8_l4096_r4: B8 L4096 H32 P64 N128 A32 R4, output norm",
                         "call_ms": cm, "main_kernel_ms": km, "tokens_per_s": Bm * Lm / (cm * 1e-3),
                         "min_flops": flops, "fp32_tflops": flops / (cm * 1e-3) / 1e12,
                         "fp32_frac": flops / (cm * 1e-3) / 1e12 / FP32_PEAK_TFLOPS, "bound": "fp32 matrix",
                         "algorithmic_bytes": byt, "gbs": byt / (cm * 1e-3) / 1e9}
    del inp, ops, ws, out


    # SISO backward at the forward's geometry: the eleven gradients from dout
    from workloads import output_gradient, preprocess_output_gradients, packed_projection
    w = WORKLOADS["siso_b4_l2048"]
    d = w.dims
    ins = {k: torch.from_numpy(v).to(dev) for k, v in ssm_inputs(d, seed=w.seed, mimo=False).items()}
    dout = torch.from_numpy(output_gradient(d, seed=w.seed)).to(dev)
    cfg = m3.SsmConfig(d.B, d.L, d.H, d.G, d.P, d.N, d.A)
    grads = {k: torch.empty_like(ins[k]) for k in ops11}
    ws = torch.empty(m3.siso_bwd_workspace_bytes(cfg), dtype=torch.uint8, device=dev)

    def one_b():
        m3.m3_siso_bwd(dout, *[ins[k] for k in ops11], cfg, grads=grads, workspace=ws)
    for _ in range(3):
        one_b()
    torch.cuda.synchronize()
    n_calls = 10
    a.record()
    for _ in range(n_calls):
        one_b()
    b.record()
    torch.cuda.synchronize()
    cm = a.elapsed_time(b) / n_calls
    Bb, Lb, Hb, Pb, Nb, Ab = d.B, d.L, d.H, d.P, d.N, d.A
    # 12 N P per token-head: the forward state update and read-out, the reverse
    # adjoint update, and the three adjoint contractions h^T gy, G^T x, G K
    flops = 12 * Nb * Pb * Bb * Lb * Hb
    # operands and dout read once, the eleven gradients written once
    byt = 4 * (2 * (2 * Bb * Lb * d.groups * Nb + 3 * Bb * Lb * Hb * Pb + 3 * Bb * Lb * Hb + Bb * Lb * Ab
                    + 2 * Hb * Nb + Hb) - Bb * Lb * Hb * Pb)
    rows["siso_bwd"] = {"workload": "siso_b4_l2048: B4 L2048 H24 P64 N128 A32, dout ~ N(0,1)",
                        "call_ms": cm, "tokens_per_s": Bb * Lb / (cm * 1e-3), "min_flops": flops,
                        "fp32_tflops": flops / (cm * 1e-3) / 1e12,
                        "fp32_frac": flops / (cm * 1e-3) / 1e12 / FP32_PEAK_TFLOPS,
                        "algorithmic_bytes": byt, "gbs": byt / (cm * 1e-3) / 1e9,
                        "hbm_frac": byt / (cm * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "workspace_bytes": ws.numel(), "calls_timed": n_calls}
    del ins, dout, grads, ws

    # MIMO backward at the MIMO scan's geometry
    w = WORKLOADS["mimo_b8_l4096_r4"]
    d = w.dims
    ins = {k: torch.from_numpy(v).to(dev) for k, v in ssm_inputs(d, seed=w.seed, dt_range=w.dt_range).items()}
    dout = torch.from_numpy(output_gradient(d, seed=w.seed)).to(dev)
    cfg = m3.SsmConfig(d.B, d.L, d.H, d.G, d.P, d.N, d.A, d.R, True, True, True)
    names15 = ops11 + ("mimo_x", "mimo_z", "mimo_o", "norm_weight")
    grads = {k: torch.empty_like(ins[k]) for k in names15}
    ws = torch.empty(m3.mimo_bwd_workspace_bytes(cfg), dtype=torch.uint8, device=dev)

    def one_mb():
        m3.m3_mimo_bwd(dout, *[ins[k] for k in names15], cfg, grads=grads, workspace=ws)
    for _ in range(2):
        one_mb()
    torch.cuda.synchronize()
    n_calls = 5
    a.record()
    for _ in range(n_calls):
        one_mb()
    b.record()
    torch.cuda.synchronize()
    mbm = a.elapsed_time(b) / n_calls
    Bm, Lm, Hm, Pm, Nm, Rm = d.B, d.L, d.H, d.P, d.N, d.R
    # 12 R N P per token-head: as the SISO backward, with the rank sums
    mflops = 12 * Rm * Nm * Pm * Bm * Lm * Hm
    rows["mimo_bwd"] = {"workload": "mimo_b8_l4096_r4: B8 L4096 H32 P64 N128 A32 R4, output norm, dout ~ N(0,1)",
                        "call_ms": mbm, "tokens_per_s": Bm * Lm / (mbm * 1e-3), "min_flops": mflops,
                        "fp32_tflops": mflops / (mbm * 1e-3) / 1e12,
                        "fp32_frac": mflops / (mbm * 1e-3) / 1e12 / FP32_PEAK_TFLOPS,
                        "workspace_bytes": ws.numel(), "calls_timed": n_calls}
    del ins, dout, grads, ws

    # preprocess backward over the [8192 x 3432] packed projection, all eight output gradients
    w = WORKLOADS["siso_b4_l2048"]
    d = w.dims
    pk = packed_projection(d, seed=w.seed)
    I, M = d.H * d.P, d.groups * d.N
    pcfg = m3.PreprocessConfig(I, d.N, d.H, d.A, d.groups, 1, 1e-5, 1e-3, 0.1, 1e-4)
    rows_n = d.B * d.L
    proj = torch.from_numpy(pk["projected"]).to(dev)
    bias = torch.from_numpy(pk["dt_bias"]).to(dev)
    pg = {k: torch.from_numpy(v).to(dev)
          for k, v in preprocess_output_gradients(rows_n, I, M, d.H, d.A, seed=w.seed).items()}
    pouts = {"projected": torch.empty_like(proj), "dt_bias": torch.empty_like(bias)}

    def one_p():
        m3.m3_preprocess_bwd(proj, bias, pcfg, pg, outs=pouts)
    for _ in range(3):
        one_p()
    torch.cuda.synchronize()
    n_calls = 20
    a.record()
    for _ in range(n_calls):
        one_p()
    b.record()
    torch.cuda.synchronize()
    pm = a.elapsed_time(b) / n_calls
    Wp = pcfg.width
    pbyt = 4 * (3 * rows_n * Wp + 2 * d.H)   # projected and the gradients read, d_projected written
    rows["preprocess_bwd"] = {"workload": "[8192 x 3432] packed projection (siso_b4_l2048 geometry)",
                              "ms": pm, "algorithmic_bytes": pbyt, "gbs": pbyt / (pm * 1e-3) / 1e9,
                              "hbm_frac": pbyt / (pm * 1e-3) / 1e9 / HBM_PEAK_GBS, "bound": "hbm",
                              "calls_timed": n_calls}
    # long-sequence SISO scan: B1 L65536 H32, dt in [1e-3, 0.01] (m3_siso_fwd on dense operands).
    # Measured last: the step's warmup then starts from the clocks the scan kernels hold.
    w = WORKLOADS["siso_long_l65536"]
    d = w.dims
    inp = {k: torch.from_numpy(v).to(dev) for k, v in ssm_inputs(d, seed=w.seed, dt_range=w.dt_range).items()}
    cfg = m3.SsmConfig(d.B, d.L, d.H, d.G, d.P, d.N, d.A)
    ws = torch.empty(max(1, m3.siso_fwd_workspace_bytes(cfg)), dtype=torch.uint8, device=dev)
    out = torch.empty(d.B, d.L, d.H, d.P, device=dev)
    ops = [inp[k] for k in ops11]
    for _ in range(5):
        m3.m3_siso_fwd(*ops, cfg, out=out, workspace=ws)
    torch.cuda.synchronize()
    kms, cms = [], []
    for _ in range(20):
        e0, e1 = new_event(), new_event()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        lib.m3_set_profile_events(e0, e1)
        a.record()
        m3.m3_siso_fwd(*ops, cfg, out=out, workspace=ws)
        b.record()
        torch.cuda.synchronize()
        lib.m3_set_profile_events(None, None)
        hip.hipEventElapsedTime(ctypes.byref(f), e0, e1)
        kms.append(f.value)
        cms.append(a.elapsed_time(b))
        hip.hipEventDestroy(e0)
        hip.hipEventDestroy(e1)
    km, cm = float(np.mean(kms)), float(np.mean(cms))
    byt = scan_algorithmic_bytes(d.B, d.L, d.H, d.groups, d.P, d.N, d.A)
    rows["siso_long_scan"] = {
        "workload": "siso_long_l65536: B1 L65536 H32 G1 P64 N128 A32, dt in [1e-3, 0.01], m3_siso_fwd",
        "call_ms": cm, "main_kernel_ms": km, "tokens_per_s": d.B * d.L / (cm * 1e-3),
        "algorithmic_bytes": byt, "bound": "hbm",
        "main_kernel": DENSE_KERNEL, "main_kernel_gbs": byt / (km * 1e-3) / 1e9,
        "main_kernel_hbm_frac": byt / (km * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "call_gbs": byt / (cm * 1e-3) / 1e9, "call_hbm_frac": byt / (cm * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "workspace_bytes": ws.numel(), "calls_timed": len(cms)}
    del inp, ops, ws, out

    return rows


def _read_csv(pattern):
    files = glob.glob(pattern, recursive=True)
    if not files:
        raise FileNotFoundError(pattern)
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def summarize(stats_dir, fetch_dir, write_dir, calib_mib):
    """Write the kernel-time summary and the counter-derived traffic of the main
    scan kernel.  FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by the
    ratio between the known size of a plain device copy and what the same
    counter reads for that copy in the same run."""
    stats = _read_csv(os.path.join(stats_dir, "**", "*kernel_stats.csv"))
    def counter(d, name):
        rows = _read_csv(os.path.join(d, "**", "*counter_collection.csv"))
        main = [float(r["Counter_Value"]) for r in rows
                if r["Counter_Name"] == name and MAIN_KERNEL in r["Kernel_Name"]]
        copy = [float(r["Counter_Value"]) for r in rows
                if r["Counter_Name"] == name and COPY_KERNEL in r["Kernel_Name"]]
        return sum(main) / len(main), sum(copy) / len(copy)
    f_main, f_copy = counter(fetch_dir, "FETCH_SIZE")
    w_main, w_copy = counter(write_dir, "WRITE_SIZE")
    known = calib_mib * 1024 * 1024
    fetch_scale = known / (f_copy * 1024.0)
    write_scale = known / (w_copy * 1024.0)
    out = {
        "kernel": MAIN_KERNEL + " (main scan pass on the packed rows)",
        "workload": "siso_b4_l2048 (B4 L2048 H24 G1 P64 N128 A32), bench.py default run",
        "kernel_source_sha256": kernel_source_hash(),
        "fetch_kib_per_dispatch": f_main, "write_kib_per_dispatch": w_main,
        "copy_mib": calib_mib, "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "fetch_bytes": f_main * 1024.0 * fetch_scale, "write_bytes": w_main * 1024.0 * write_scale,
        "kernel_stats": [{k: r[k] for k in ("Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage")}
                         for r in stats],
    }
    out["traffic_bytes"] = out["fetch_bytes"] + out["write_bytes"]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: v for k, v in out.items() if k != "kernel_stats"}, indent=1))
    return 0


def recorded_traffic():
    """Counter-derived HBM bytes of the main kernel, if taken from the current source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash() or not rec.get("kernel", "").startswith(MAIN_KERNEL):
        return None
    return rec.get("traffic_bytes")


def scan_algorithmic_bytes(B, L, H, G, P, N, A) -> int:
    """Each scan operand read once, out written once (fp32)."""
    elems = 3 * B * L * H * P + 2 * B * L * G * N + 3 * B * L * H + B * L * A + 2 * H * N + H
    return 4 * elems


def preprocess_algorithmic_bytes(rows, W, I, M, H, A) -> int:
    """Packed row and dt_bias read once, the eight outputs written once."""
    return 4 * (rows * W + H + rows * (2 * I + 2 * M + 3 * H + A))


def main():
    args = parse()
    if args.summarize:
        return summarize(*args.summarize, args.calib_mib)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: every (batch, head) "
              "chain is independent, so more GPUs would shard batch/heads with no communication.",
              file=sys.stderr)
        return 2

    import torch
    import selective_state_space_mamba3_amd as m3
    from selective_state_space_mamba3_amd import _binding as bd
    from workloads import WORKLOADS, packed_projection

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 3
    lib = m3.lib()  # raises if libm3.so is missing: there is no CPU fallback
    dev = torch.device("cuda:0")
    w = WORKLOADS["siso_b4_l2048"]
    d = w.dims
    B, L, H, G, P, N, A = d.B, d.L, d.H, d.groups, d.P, d.N, d.A
    rows, I, M = B * L, H * P, G * N
    pcfg = m3.PreprocessConfig(inner_size=I, state_size=N, num_heads=H, num_rope_angles=A, num_groups=G,
                               mimo_rank=1, epsilon=1e-5, dt_min=1e-3, dt_max=0.1, a_floor=1e-4)
    scfg = m3.SsmConfig(B, L, H, G, P, N, A, 1, True, True, False)
    W = pcfg.width

    # ---- inputs resident in HBM -------------------------------------------
    host_sets, sets = [], []
    for k in range(args.sets):
        hs = packed_projection(d, seed=w.seed + 100 * k, dt_range=w.dt_range)
        host_sets.append(hs if k == 0 else None)
        ds = {key: torch.from_numpy(v).to(dev) for key, v in hs.items()}
        outs = {"x": torch.empty(rows, I, device=dev), "z": torch.empty(rows, I, device=dev),
                "bh": torch.empty(rows, M, device=dev), "ch": torch.empty(rows, M, device=dev),
                "dt": torch.empty(rows, H, device=dev), "adt": torch.empty(rows, H, device=dev),
                "trap": torch.empty(rows, H, device=dev), "angle": torch.empty(rows, A, device=dev)}
        ds["pre"] = outs
        ds["out"] = torch.empty(B, L, H, P, device=dev)
        ds["out2"] = torch.empty(B, L, H, P, device=dev)
        sets.append(ds)
    ws = torch.empty(max(1, m3.siso_fwd_workspace_bytes(scfg)), dtype=torch.uint8, device=dev)

    def scan_operands(s):
        o = s["pre"]
        return (o["ch"].view(B, L, G, N), o["bh"].view(B, L, G, N), o["x"].view(B, L, H, P),
                o["z"].view(B, L, H, P), o["adt"].view(B, L, H), o["dt"].view(B, L, H),
                o["trap"].view(B, L, H), o["angle"].view(B, L, A), s["c_bias"], s["b_bias"], s["d"])

    fws = torch.empty(max(1, m3.siso_fwd_packed_workspace_bytes(pcfg, scfg)), dtype=torch.uint8, device=dev)

    def step(s):
        """The bench step: preprocess fused into the scan, one call on the packed rows."""
        m3.m3_siso_fwd_packed(s["projected"], s["dt_bias"], s["c_bias"], s["b_bias"], s["d"], pcfg, scfg,
                              out=s["out"], workspace=fws)

    def two_call(s, ev=None):
        """The same pass as two calls: m3_preprocess, then m3_siso_fwd on its outputs."""
        if ev is not None:
            ev[0].record()
        m3.m3_preprocess(s["projected"], s["dt_bias"], pcfg, outs=s["pre"])
        if ev is not None:
            ev[1].record()
        m3.m3_siso_fwd(*scan_operands(s), scfg, out=s["out2"], workspace=ws)
        if ev is not None:
            ev[2].record()

    # ---- parity in the same run, before timing ----------------------------
    parity = None
    if not args.no_parity:
        import oracle as O
        s0 = sets[0]
        step(s0)
        two_call(s0)
        torch.cuda.synchronize()
        same = bool(torch.equal(s0["out"], s0["out2"]))
        hs = host_sets[0]
        ocfg = O.PreprocessConfig(I, N, H, A, G, 1, 1e-5, 1e-3, 0.1, 1e-4)
        pre = O.preprocess(hs["projected"], hs["dt_bias"], ocfg)
        heads = [0, H - 1]
        shp = {"x": (B, L, H, P), "z": (B, L, H, P), "bh": (B, L, G, N), "ch": (B, L, G, N),
               "dt": (B, L, H), "adt": (B, L, H), "trap": (B, L, H), "angle": (B, L, A)}
        oi = {k: pre[k].reshape(shp[k]) for k in shp}
        ref = O.siso_scan(oi["ch"], oi["bh"], oi["x"], oi["z"], oi["adt"], oi["dt"], oi["trap"], oi["angle"],
                          hs["c_bias"], hs["b_bias"], hs["d"], O.SsmConfig(B, L, H, G, P, N, A), heads=heads)
        got = s0["out"].cpu().numpy()[:, :, heads]
        e = O.parity_error(got, ref)
        parity = {"e": e["e"], "tol": 1e-4, "sample": f"all batch rows of heads {heads}, full sequence",
                  "pass": bool(e["e"] <= 1e-4 and e["nonfinite"] == 0 and same),
                  "two_call_bit_identical": same}
        if not parity["pass"]:
            print(json.dumps({"parity_failed": parity}), file=sys.stderr)
            return 4

    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.m3_set_profile_events.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    # Events for timing only: without the system-scope fence that a default
    # event adds when it is recorded (an L2 writeback and invalidate between
    # the kernels it separates); the elapsed times are read after a device
    # synchronisation.
    HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000

    def new_event():
        e = ctypes.c_void_p()
        if hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(HIP_EVENT_DISABLE_SYSTEM_FENCE)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e

    class FenceFreeEvent:
        """A timing event of that kind recorded on torch's current stream."""

        def __init__(self):
            self.e = new_event()

        def record(self):
            if hip.hipEventRecord(self.e, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) != 0:
                raise RuntimeError("hipEventRecord failed")

        def elapsed_time(self, other):
            f = ctypes.c_float()
            if hip.hipEventElapsedTime(ctypes.byref(f), self.e, other.e) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            return f.value

    # ---- the other rows, each at its own workload --------------------------
    # (measured first: seconds of GPU work that leave the GPU at the clocks it
    # holds under load, so that a short warmup suffices before the timed steps)
    rows_out = None
    if not args.no_rows:
        rows_out = measure_rows(torch, m3, lib, hip, new_event, dev)
        torch.cuda.empty_cache()

    # ---- warmup ------------------------------------------------------------
    for i in range(args.warmup):
        step(sets[i % len(sets)])
        two_call(sets[i % len(sets)])
    torch.cuda.synchronize()

    # ---- timed region ------------------------------------------------------
    # The library records the main pass's events on every KERN_EVERY-th timed
    # step only: each recorded event leaves the GPU idle for about 4.5 us
    # between the kernels it separates (kernel trace), which would otherwise
    # add about 9 us to every step.
    K = args.steps
    KERN_EVERY = 4
    kern_steps = [i for i in range(K) if i % KERN_EVERY == KERN_EVERY - 1] or [K - 1]
    kern_ev = {i: (new_event(), new_event()) for i in kern_steps}
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_begin.record()
    for i in range(K):
        if i in kern_ev:
            lib.m3_set_profile_events(kern_ev[i][0], kern_ev[i][1])
        else:
            lib.m3_set_profile_events(None, None)
        step(sets[i % len(sets)])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    lib.m3_set_profile_events(None, None)

    # the two-call form of the same pass, after the timed region: timed as a
    # whole with no events between its calls, then once more with events
    # for its breakdown and the dense main pass's time
    t2_begin = torch.cuda.Event(enable_timing=True)
    t2_end = torch.cuda.Event(enable_timing=True)
    t2_begin.record()
    for i in range(K):
        two_call(sets[i % len(sets)])
    t2_end.record()
    torch.cuda.synchronize()
    dense_ev = [(new_event(), new_event()) for _ in range(K)]
    step_ev = [[FenceFreeEvent() for _ in range(3)] for _ in range(K)]
    for i in range(K):
        lib.m3_set_profile_events(dense_ev[i][0], dense_ev[i][1])
        two_call(sets[i % len(sets)], step_ev[i])
    torch.cuda.synchronize()
    lib.m3_set_profile_events(None, None)

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * 1024 * 1024 // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty(n, device=dev)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ms_total = t_begin.elapsed_time(t_end)
    ms_step = ms_total / K
    f = ctypes.c_float()

    def event_ms(pairs):
        out = []
        for a, b in pairs:
            hip.hipEventElapsedTime(ctypes.byref(f), a, b)
            out.append(f.value)
            hip.hipEventDestroy(a)
            hip.hipEventDestroy(b)
        return float(np.mean(out))
    kern_avg = event_ms(kern_ev.values())
    dense_avg = event_ms(dense_ev)
    pre_ms = [ev[0].elapsed_time(ev[1]) for ev in step_ev]
    scan_ms = [ev[1].elapsed_time(ev[2]) for ev in step_ev]
    two_ms = t2_begin.elapsed_time(t2_end) / K
    tokens = B * L
    scan_bytes = scan_algorithmic_bytes(B, L, H, G, P, N, A)
    pre_bytes = preprocess_algorithmic_bytes(rows, W, I, M, H, A)
    # the fused step: packed rows and dt_bias read once, biases and D read, out written once
    step_bytes = 4 * (rows * W + H + 2 * H * N + H + B * L * H * P)
    min_flops = 4 * N * P * B * L * H  # state read-out and state update, per token-head
    kern_gbs = scan_bytes / (kern_avg * 1e-3) / 1e9
    scan_call_ms = float(np.mean(scan_ms))
    pre_avg = float(np.mean(pre_ms))

    # ---- CPU baseline: the float64 oracle on the host cores ---------------
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        # every core: the 24 heads sharded over processes, each with the preprocess
        n_proc, crit, t_pre_med, per_shard = oracle_all_cores(H)
        # one thread: the preprocess and a sample of heads, scaled to all heads
        hsel = list(range(min(args.cpu_heads, H)))
        with threadpool_limits(limits=1):
            t_pre, t_scan = _oracle_pass(host_sets[0], hsel)
        est = t_pre + t_scan * H / len(hsel)
        cpu = {"value": tokens / crit, "unit": "tokens/s", "cores": n_proc, "kind": "oracle",
               "sample": (f"float64 oracle on the whole step's work: preprocess of all {rows} packed rows and "
                          f"the scan of all {H} heads over all {B} batch rows and {L} tokens, heads sharded "
                          f"over {n_proc} processes of one thread (at most {per_shard} heads each; every "
                          f"process repeats the preprocess, median {t_pre_med:.2f} s); time = slowest "
                          f"process, {crit:.2f} s"),
               "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
               "one_thread": {"value": tokens / est, "unit": "tokens/s", "cores": 1,
                              "sample": (f"preprocess of all {rows} rows ({t_pre:.2f} s) + scan of "
                                         f"{len(hsel)} of {H} heads ({t_scan:.2f} s), scan time scaled by "
                                         f"{H}/{len(hsel)}")}}
        if args.cpu_decode_steps > 0 and not args.no_rows:
            cpu["rows"] = oracle_rows_all_cores(args.cpu_decode_steps)

    result = {
        "metric": "scan fwd tokens/s + HBM GB/s (% roofline), SISO B4 L2048 H24 P64 N128",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "arithmetic": "fp32 storage, accumulation and element-wise work; in the main pass S = Q K^T, the "
                      "read-out Q h'^T and the state update K^T (w x) as fp16 matrix products of "
                      "power-of-two-scaled head/tail splits (about 2^-21 per product), M X in fp32; in the "
                      "segment-summary pass the state update as bf16 matrix products of six-term splits "
                      "(about 2^-23 per product)",
        "data": "synthetic",
        "config": {"workload": "siso_b4_l2048: m3_siso_fwd_packed on the [8192 x 3432] packed projection "
                               "(preprocess fused into the scan)",
                   "batch": B, "seq_len": L, "heads": H, "groups": G, "head_dim": P, "state": N,
                   "rope_angles": A, "has_z": True, "has_d": True, "input_sets": args.sets},
        "roofline": {"bound": "hbm", "achieved": kern_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": kern_gbs / HBM_PEAK_GBS, "traffic": recorded_traffic(),
                     "kernel": MAIN_KERNEL + " (main scan pass on the packed rows)",
                     "kernel_ms": kern_avg, "kernel_launches_timed": len(kern_steps), "algorithmic_bytes": scan_bytes,
                     "fp32_tflops_min_work": min_flops / (kern_avg * 1e-3) / 1e12,
                     "fp32_frac": min_flops / (kern_avg * 1e-3) / 1e12 / FP32_PEAK_TFLOPS,
                     # the same bytes over the whole scan call (summary pass, fold and
                     # main pass; the two-call form's m3_siso_fwd) and over the whole step
                     "scan_level": {"ms": scan_call_ms, "gbs": scan_bytes / (scan_call_ms * 1e-3) / 1e9,
                                    "frac": scan_bytes / (scan_call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                    "what": "m3_siso_fwd call on dense operands: summary pass + main pass"},
                     "step_level": {"ms": ms_step, "algorithmic_bytes": step_bytes,
                                    "gbs": step_bytes / (ms_step * 1e-3) / 1e9,
                                    "frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                    "what": "the timed step: packed rows read once, out written once"}},
        "two_call_step": {"ms": two_ms, "tokens_per_s": tokens / (two_ms * 1e-3),
                          "calls": "m3_preprocess then m3_siso_fwd", "main_kernel": DENSE_KERNEL,
                          "main_kernel_ms": dense_avg, "main_kernel_gbs": scan_bytes / (dense_avg * 1e-3) / 1e9,
                          "main_kernel_hbm_frac": scan_bytes / (dense_avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "steps_timed": K},
        "scan": {"call_ms": scan_call_ms, "tokens_per_s": tokens / (scan_call_ms * 1e-3),
                 "gbs": scan_bytes / (scan_call_ms * 1e-3) / 1e9,
                 "hbm_frac": scan_bytes / (scan_call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "workspace_bytes": m3.siso_fwd_workspace_bytes(scfg)},
        "preprocess": {"ms": pre_avg, "algorithmic_bytes": pre_bytes,
                       "gbs": pre_bytes / (pre_avg * 1e-3) / 1e9,
                       "hbm_frac": pre_bytes / (pre_avg * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "wall_s_timed": wall,
        "parity": parity,
        "rows": rows_out,
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
