"""Benchmark of the multi-scale deformable attention hot path on one MI355X.

One step = one forward (msda_forward) plus one backward (msda_backward, all
three gradients) over the encoder-shaped workload: B=2, four levels
(100,167),(50,84),(25,42),(13,21) so L = N_q = 22223, N_h=8, C_h=32, N_p=4,
float32, BLNC / BQHLP2, zeros padding, align_corners off; locations
U[-0.05, 1.05], softmax attention weights, grad_output ~ N(0, 1). Inputs are
seeded, synthetic, and resident in HBM before the timed region starts.

Prints ONE JSON line. `value` is queries/s of whole steps. `roofline` prices
the dominant launch (the backward call) against the ceiling of the memory
level that serves its gathers: the L2 -> CU path (8 XCDs x 16 L2 channels x
128 B per clock x 2.4 GHz), measured beside it with the probe library's
L2-resident read probes; HBM traffic from calibration-free rocprofv3 counters
(committed summary) is reported beside it against the 8 TB/s HBM peak.
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same
workload on this host's cores (and on one core).

`--report` instead times every named workload (forward, and backward where it
has a grad_output) warm and with cold caches, next to the CPU oracle on all
host cores and on one core, and prints one JSON line per workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E peak, GB/s
MFMA_F32_PEAK_TFLOPS = 157.3    # MI355X dense float32 matrix-core peak, TFLOP/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bfloat16 matrix-core peak, TFLOP/s
# L2 -> CU read ceiling: 8 XCDs, each with a 16-channel L2 that returns one
# 128-byte line per channel per clock, at the 2.4 GHz peak engine clock
# (the same figure as 256 CUs x 64 B per clock of vector-memory return).
XCDS, L2_CHANNELS_PER_XCD, L2_BYTES_PER_CLOCK, CLOCK_GHZ = 8, 16, 128, 2.4
L2_PEAK_GBS = XCDS * L2_CHANNELS_PER_XCD * L2_BYTES_PER_CLOCK * CLOCK_GHZ   # 39,321.6 GB/s
PROBE_LIB = os.path.join(ROOT, "scale_deformable_attention_forward_amd", "libmsda_probe.so")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "msda_encoder_fp32_fwd_bwd_hbm_traffic.txt")
METRIC = "queries/s and effective gathered HBM GB/s (% of peak), fwd+bwd, 1 MI355X"
WORKLOAD_NUM = 5                # encoder shapes with grad_output (the forward uses the same arrays)
BACKWARD_KERNELS = ("backward_fast_kernel", "band_count_kernel", "band_scan_kernel", "band_fill_kernel",
                    "tile_scatter_kernel", "band_reduce_kernel")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU oracle sample time")
    ap.add_argument("--quick", action="store_true",
                    help="only the timed steps (no cold-cache timings, probes or CPU oracle): for profiler runs")
    ap.add_argument("--workload", type=int, default=WORKLOAD_NUM,
                    help="named workload whose forward+backward a step runs (default: the encoder shape); "
                         "workloads without a grad_output get one drawn with seed 1000 + workload number")
    ap.add_argument("--mode-variants", action="store_true",
                    help="time forward and backward at the square bf16 workload's shapes with one of its "
                         "modes (padding, location range, dtype, layouts, align_corners) changed at a time")
    ap.add_argument("--generic-backward", action="store_true",
                    help="only time the backward's generic path (float atomics into grad_value) at the "
                         "encoder shape: grad_value is a view one element off 16-byte alignment")
    ap.add_argument("--report", action="store_true",
                    help="time every named workload (GPU warm/cold, CPU oracle all cores / 1 core)")
    ap.add_argument("--producer", action="store_true",
                    help="time the producer of locations and weights (projection + softmax), alone, fused "
                         "with the sampler, and its backward, at the encoder shape with D=256")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (HBM counter calibration)")
    return ap.parse_args()


# ------------------------------------------------------------ byte counts ---

def _loc_bqhlp2(d):
    loc = d["sampling_locations"]
    if d["sampling_locations_layout"] == "B2QHLP":
        loc = np.moveaxis(loc, 1, -1)
    return loc


def counted_corners(d):
    """(sample, corner) pairs the method must read: corner index inside its
    level and bilinear weight nonzero (float32 coordinate map and border clamp
    as in the kernels). Counted in numpy; independent of the GPU path."""
    loc = _loc_bqhlp2(d)
    align, border = bool(d["align_corners"]), d["padding_mode"] == "border"
    n = 0
    for l, (H, W) in enumerate(d["spatial_shapes"]):
        ux = loc[:, :, :, l, :, 0].astype(np.float64)
        uy = loc[:, :, :, l, :, 1].astype(np.float64)
        if align:
            x = (ux.astype(np.float32) * np.float32(W - 1)).astype(np.float32)
            y = (uy.astype(np.float32) * np.float32(H - 1)).astype(np.float32)
        else:   # u*W - 0.5 is exact in float64 here; one rounding to float32 = fmaf
            x = (ux * W - 0.5).astype(np.float32)
            y = (uy * H - 0.5).astype(np.float32)
        if border:
            x = np.clip(x, 0, W - 1)
            y = np.clip(y, 0, H - 1)
        x0, y0 = np.floor(x), np.floor(y)
        fx, fy = x - x0, y - y0
        x0, y0 = x0.astype(np.int64), y0.astype(np.int64)
        for dx, wx in ((0, 1.0 - fx), (1, fx)):
            okx = (x0 + dx >= 0) & (x0 + dx < W) & (wx != 0)
            for dy, wy in ((0, 1.0 - fy), (1, fy)):
                n += int((okx & (y0 + dy >= 0) & (y0 + dy < H) & (wy != 0)).sum())
    return n


def byte_counts(d):
    """Algorithmic bytes per launch: nominal (4 corners per sample) and counted
    (corners the method must read), plus the streams each launch reads or
    writes once."""
    B, N_q, N_h, N_l, N_p = d["attention_weights"].shape
    C_h = d["value"].shape[-1]
    s_v = 2 if d["value_dtype"] == "bf16" else 4
    samples = B * N_q * N_h * N_l * N_p
    corner_bytes = C_h * s_v
    cnt = counted_corners(d)
    loc_b, attn_b = samples * 8, samples * 4
    out_b = B * N_q * N_h * C_h * s_v
    value_b = d["value"].size * s_v
    fwd_streams = loc_b + attn_b + out_b
    # backward: grad_output + loc + attn in, grad_loc + grad_attn out, grad_value written once
    bwd_streams = out_b + loc_b + attn_b + loc_b + attn_b + value_b
    return {
        "samples": samples,
        "counted_corners": cnt,
        "counted_fraction": cnt / (4 * samples),
        "forward": {"nominal": 4 * samples * corner_bytes + fwd_streams,
                    "counted": cnt * corner_bytes + fwd_streams},
        # re-gather + scatter (read-modify-write counted once)
        "backward": {"nominal": 2 * 4 * samples * corner_bytes + bwd_streams,
                     "counted": 2 * cnt * corner_bytes + bwd_streams},
        "queries": B * N_q,
    }


def measured_traffic():
    """Memory-side bytes per forward launch and per backward call from the
    committed rocprofv3 counter summary: reads = FETCH_SIZE scaled by what it
    reads on a plain 1 GiB device copy (x 2.0 on this part), writes =
    WRITE_SIZE (TCC_EA0_WRREQ in 32- and 64-byte units, exact on the copy).
    The reads agree within 0.4% with 32 x TCC_EA0_RDREQ_DRAM_32B (the L2's
    read requests to memory in 32-byte units), which is used where FETCH_SIZE
    was not taken (the generic path) and reported beside it. Also each
    kernel's L2 hit rate and atomic request counts. (None, None, {}) when a
    kernel source changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None, None, {}
    for rel, digest in rec["sources_sha256"].items():
        path = os.path.join(ROOT, rel)
        if not os.path.exists(path) or hashlib.sha256(open(path, "rb").read()).hexdigest() != digest:
            return None, None, {}
    fwd = bwd = 0.0
    per = {}
    for name, c in rec["per_dispatch"].items():
        n = c["dispatches_per_call"]
        rd = c.get("fetch_bytes_copy_scaled", c["read_bytes"])
        b = (rd + c["write_bytes"]) * n
        per[name] = {"hbm_bytes_per_call": b, "read_bytes_per_call": rd * n,
                     "read_bytes_request_counter_per_call": c["read_bytes"] * n,
                     "write_bytes_per_call": c["write_bytes"] * n, "l2_hit_pct": c.get("L2_hit_pct"),
                     "tcc_atomic_per_call": c.get("TCC_ATOMIC", 0.0) * n}
        if name.startswith("forward_kernel"):
            fwd += b
        elif c.get("path", "tiled") == "tiled":
            bwd += b
    return fwd, bwd, per


def compulsory_bytes(d):
    """Bytes every launch must move to or from memory at least once: its
    inputs read and outputs written (value read once however often it is
    gathered)."""
    B, N_q, N_h, N_l, N_p = d["attention_weights"].shape
    C_h = d["value"].shape[-1]
    s_v = 2 if d["value_dtype"] == "bf16" else 4
    samples = B * N_q * N_h * N_l * N_p
    value_b = d["value"].size * s_v
    out_b = B * N_q * N_h * C_h * s_v
    loc_b, attn_b = samples * 8, samples * 4
    return {"forward": value_b + loc_b + attn_b + out_b,
            # grad_output, value, loc, attn in; grad_value, grad_loc, grad_attn out
            "backward": out_b + value_b + loc_b + attn_b + value_b + loc_b + attn_b}


def probe_ceilings(dev, stream):
    """Read rates (GB/s) the probe library reaches on this GPU: the vector L1,
    an L2-resident stream, L2-resident 128-byte rows at random (the gathers'
    access shape) and an HBM stream; median of 5 timed launches each."""
    import ctypes
    import torch
    if not os.path.exists(PROBE_LIB):
        raise ImportError(f"{PROBE_LIB} is not built: run `python -m scale_deformable_attention_forward_amd.build`")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.msda_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.msda_probe_read.restype = ctypes.c_int
    lib.msda_probe_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.msda_probe_bytes.restype = ctypes.c_int64
    blocks = 2048
    buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)     # 1 GiB
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    cases = (("vector_l1", 0, 16 << 10, 4000), ("l2_stream", 1, 2 << 20, 1000),
             ("l2_gather_128B_rows", 2, 2 << 20, 1000), ("hbm_stream", 3, 1 << 30, 150))
    res = {}
    for name, mode, span, iters in cases:
        nbytes = lib.msda_probe_bytes(mode, blocks, iters)

        def launch():
            rc = lib.msda_probe_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * 4, span, mode, blocks, iters,
                                     ctypes.c_void_p(sink.data_ptr()), sp)
            if rc != 0:
                raise RuntimeError(f"probe {name}: msda_probe_read returned {rc}")
        ms = time_launches(launch, stream, 5, 2)
        res[name] = nbytes / (float(np.median(ms)) * 1e-3) / 1e9
    del buf, sink
    return res


# ------------------------------------------------------------------ timing ---

def time_launches(fn, stream, iters, warmup, cold_buf=None):
    """Per-launch durations (ms) from HIP events recorded on `stream` around
    each launch; with cold_buf, the buffer is overwritten before every launch
    (outside the events) to evict L2 and the Infinity Cache."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i in range(iters):
        if cold_buf is not None:
            cold_buf.fill_(float(i))
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def stats(ms):
    return {"ms_mean": float(np.mean(ms)), "ms_median": float(np.median(ms)), "ms_max": float(np.max(ms)),
            "ms_p10": float(np.percentile(ms, 10)), "ms_p90": float(np.percentile(ms, 90))}


def _device_inputs(d, dev):
    import torch
    t = {}
    if d["value_dtype"] == "bf16":
        t["value"] = torch.from_numpy(d["value_bf16_bits"].view(np.int16).copy()).view(torch.bfloat16).to(dev)
    else:
        t["value"] = torch.from_numpy(d["value"]).to(dev)
    t["loc"] = torch.from_numpy(d["sampling_locations"]).to(dev)
    t["attn"] = torch.from_numpy(d["attention_weights"]).to(dev)
    if "grad_output" in d:
        g = torch.from_numpy(d["grad_output"]).to(dev)
        t["gout"] = g.to(torch.bfloat16) if d["value_dtype"] == "bf16" else g
    return t


def _launchers(d, t, stream):
    """forward() and (if the workload has a grad_output) backward() closures
    over pre-allocated outputs and workspace."""
    import torch
    from scale_deformable_attention_forward_amd import binding
    ss, ls = d["spatial_shapes"], d["level_start_index"]
    mode = (d["value_layout"], d["sampling_locations_layout"], d["align_corners"], d["padding_mode"])
    B, N_q = d["attention_weights"].shape[:2]
    N_h, C_h = d["attention_weights"].shape[2], d["value"].shape[-1]
    out = torch.empty((B, N_q, N_h * C_h), dtype=t["value"].dtype, device=t["value"].device)

    def fwd():
        binding.msda_forward(t["value"], ss, ls, t["loc"], t["attn"], *mode, output=out, stream=stream)

    bwd = None
    if "gout" in t:
        gv, gl, ga = torch.empty_like(t["value"]), torch.empty_like(t["loc"]), torch.empty_like(t["attn"])
        nws = binding.backward_workspace_bytes(t["value"], ss, ls, t["loc"], *mode)
        ws = torch.empty(max(1, nws), dtype=torch.uint8, device=t["value"].device)

        def bwd():
            binding.msda_backward(t["gout"], t["value"], ss, ls, t["loc"], t["attn"], *mode, grad_value=gv,
                                  grad_sampling_locations=gl, grad_attention_weights=ga, workspace=ws,
                                  stream=stream)
    return fwd, bwd


# ------------------------------------------------------------ CPU oracle ---

def _query_slice(d, nq):
    """The first nq queries of a workload (same value pyramid)."""
    s = dict(d)
    s["attention_weights"] = d["attention_weights"][:, :nq]
    if d["sampling_locations_layout"] == "B2QHLP":
        s["sampling_locations"] = d["sampling_locations"][:, :, :nq]
    else:
        s["sampling_locations"] = d["sampling_locations"][:, :nq]
    if "grad_output" in d:
        s["grad_output"] = d["grad_output"][:, :nq]
    return s


def oracle_rate(d, passes, target_s, threads=None):
    """Queries/s of the CPU oracle (fp64 C, OpenMP) running `passes` over
    growing query slices of the workload until about target_s seconds; returns
    (queries/s, threads used, description of the sample)."""
    import oracle
    prev = oracle.max_threads()
    if threads is not None:
        oracle.set_threads(threads)
    used = oracle.max_threads()
    B, N_q = d["attention_weights"].shape[:2]
    args = dict(spatial_shapes=d["spatial_shapes"], level_start_index=d["level_start_index"],
                value_layout=d["value_layout"], sampling_locations_layout=d["sampling_locations_layout"],
                align_corners=d["align_corners"], padding_mode=d["padding_mode"])
    nq, done_q, el = min(N_q, 64), 0, 0.0
    while el < target_s:
        s = _query_slice(d, nq)
        t0 = time.perf_counter()
        if "forward" in passes:
            oracle.forward(d["value"], sampling_locations=s["sampling_locations"],
                           attention_weights=s["attention_weights"], **args)
        if "backward" in passes:
            oracle.backward(s["grad_output"], d["value"], sampling_locations=s["sampling_locations"],
                            attention_weights=s["attention_weights"], **args)
        el += time.perf_counter() - t0
        done_q += B * nq
        if nq < N_q:
            nq = min(N_q, nq * 4)
    oracle.set_threads(prev)
    return done_q / el, used, f"{done_q} queries of the workload ({'+'.join(passes)}, first-query slices " \
                              f"up to the full N_q, {el:.1f} s), fp64 C oracle with OpenMP"


def cpu_baseline(d, target_s):
    """The CPU oracle on the same inputs: whole forward+backward steps on every
    core this process may run on (os.sched_getaffinity), repeated until about
    target_s seconds have run; then forward+backward on one core over
    first-query slices of the workload for about a third of that."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    prev = oracle.max_threads()
    args = (d["spatial_shapes"], d["level_start_index"])
    B, N_q = d["attention_weights"].shape[:2]
    oracle.set_threads(cores)
    try:
        used = oracle.max_threads()
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.forward(d["value"], *args, d["sampling_locations"], d["attention_weights"])
            oracle.backward(d["grad_output"], d["value"], *args, d["sampling_locations"],
                            d["attention_weights"])
            reps += 1
            el = time.perf_counter() - t0
            if el >= target_s or reps >= 50:
                break
    finally:
        oracle.set_threads(prev)
    q1, c1, s1 = oracle_rate(d, ("forward", "backward"), target_s / 3, threads=1)
    return {"value": reps * B * N_q / el, "unit": "queries/s", "cores": used,
            "kind": "oracle",
            "sample": f"{reps} full forward+backward step(s) of the same workload ({reps * B * N_q} "
                      f"queries, {el:.1f} s), fp64 C oracle with OpenMP on the {cores} cores of this "
                      "process's CPU affinity mask",
            "one_core": {"value": q1, "unit": "queries/s", "cores": c1, "sample": s1}}


# ---------------------------------------------------------------- report ---

def report(a):
    import torch
    from scale_deformable_attention_forward_amd import binding
    from scale_deformable_attention_forward_amd.workloads import WORKLOADS, make_inputs, make_workload
    binding.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    for num, wl in sorted(WORKLOADS.items()):
        d = make_workload(num)
        if "grad_output" not in d:
            # backward timing on the same arrays, with a grad_output of its own seed
            g = make_inputs(wl.B, wl.levels, wl.num_queries, wl.N_h, wl.C_h, wl.N_p, wl.seed,
                            loc_dist=wl.loc_dist, loc_range=wl.loc_range, value_dtype=wl.value_dtype,
                            value_layout=wl.value_layout, sampling_locations_layout=wl.sampling_locations_layout,
                            grad_seed=1000 + num)
            d["grad_output"] = g["grad_output"]
        t = _device_inputs(d, dev)
        fwd, bwd = _launchers(d, t, stream)
        bc = byte_counts(d)
        line = {"workload": num, "name": wl.name, "queries": bc["queries"],
                "counted_corner_fraction": bc["counted_fraction"], "dtype": wl.value_dtype}
        for name, fn in (("forward", fwd), ("backward", bwd)):
            warm = time_launches(fn, stream, a.steps, a.warmup)
            cold = time_launches(fn, stream, min(a.steps, 30), 2, cold_buf=scratch)
            avg_s = float(np.mean(warm)) * 1e-3
            line[name] = {
                "warm": stats(warm), "cold": stats(cold),
                "queries_per_s": bc["queries"] / avg_s,
                "gbs_counted": bc[name]["counted"] / avg_s / 1e9,
                "gbs_nominal": bc[name]["nominal"] / avg_s / 1e9,
                "l2_frac_counted": bc[name]["counted"] / avg_s / 1e9 / L2_PEAK_GBS,
                "effective_gbs_vs_hbm_peak": bc[name]["counted"] / avg_s / 1e9 / HBM_PEAK_GBS,
            }
        if not a.no_cpu_baseline:
            for name in ("forward", "backward"):
                tgt = a.cpu_seconds / 4
                qa, ca, sa = oracle_rate(d, (name,), tgt, threads=len(os.sched_getaffinity(0)))
                q1, c1, s1 = oracle_rate(d, (name,), tgt, threads=1)
                line[name]["cpu_oracle"] = {"all_cores": {"queries_per_s": qa, "cores": ca, "sample": sa},
                                            "one_core": {"queries_per_s": q1, "cores": c1, "sample": s1}}
        print(json.dumps(line), flush=True)


# --------------------------------------------------------------- producer ---

def producer_workspace_bytes(binding, q, w, ss, ls):
    import ctypes
    lib = binding.load_library()
    L = sum(h * wd for h, wd in ss)
    prob, keep = binding.make_problem(w["B"], L, w["N_q"], w["N_h"], 1, ss, ls, w["N_p"], value_dtype=q.dtype)
    n = ctypes.c_size_t(0)
    assert lib.msda_producer_backward_workspace_size(ctypes.byref(prob), w["D"], ctypes.byref(n)) == 0
    return max(1, n.value)


def producer_report(a):
    """One JSON line per input dtype: the producer forward, the fused producer
    + sampler against the two-call chain, and the producer backward, with
    FLOP/s against the peak of the matrix cores each one runs on (the
    forward's projection takes bfloat16 operands as they are; the backward's
    products involve float32 gradients, so they run in float32), the
    forward's memory-side bytes against the HBM peak, and the CPU oracle
    (float64 numpy) on a bounded slice of rows."""
    import torch
    import oracle.producer as oprod
    from scale_deformable_attention_forward_amd import binding
    from scale_deformable_attention_forward_amd.workloads import (PRODUCER_WORKLOAD, make_inputs,
                                                                  make_producer_inputs)
    binding.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    w = PRODUCER_WORKLOAD
    S = len(w["levels"]) * w["N_p"]
    M = w["B"] * w["N_q"]
    gemm_flop = 2.0 * M * 3 * w["N_h"] * S * w["D"]
    for dtype in ("fp32", "bf16"):
        p = make_producer_inputs(w["B"], w["levels"], w["N_q"], w["N_h"], w["N_p"], w["D"], w["seed"],
                                 value_dtype=dtype, grad_seed=w["seed"] + 1)
        v = make_inputs(w["B"], w["levels"], w["N_q"], w["N_h"], w["C_h"], w["N_p"], w["seed"] + 2,
                        value_dtype=dtype)

        def dev_t(k, src):
            if dtype == "bf16" and k + "_bf16_bits" in src:
                return torch.from_numpy(src[k + "_bf16_bits"].view(np.int16).copy()).view(torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(src[k])).to(dev)

        q, ref, wo, bo, wa, ba = (dev_t(k, p) for k in ("query", "reference_points", "offset_weight",
                                                        "offset_bias", "attention_weight", "attention_bias"))
        val = dev_t("value", v)
        ss, ls = p["spatial_shapes"], p["level_start_index"]
        loc, attn = binding.msda_producer_forward(q, ref, wo, bo, wa, ba, ss, ls, w["N_h"])
        out = torch.empty((w["B"], w["N_q"], w["N_h"] * w["C_h"]), dtype=val.dtype, device=dev)
        gl = dev_t("grad_sampling_locations", p)
        ga = dev_t("grad_attention_weights", p)
        grads = binding.msda_producer_backward(q, wo, wa, attn, gl, ga, ss, ls)   # outputs reused below
        pws = torch.empty(producer_workspace_bytes(binding, q, w, ss, ls), dtype=torch.uint8, device=dev)
        fns = {
            "forward": lambda: binding.msda_producer_forward(q, ref, wo, bo, wa, ba, ss, ls, w["N_h"],
                                                             sampling_locations=loc, attention_weights=attn,
                                                             stream=stream),
            "sampler": lambda: binding.msda_forward(val, ss, ls, loc, attn, output=out, stream=stream),
            "fused_forward": lambda: binding.msda_fused_forward(val, ss, ls, q, ref, wo, bo, wa, ba,
                                                                output=out, stream=stream),
            "backward": lambda: binding.msda_producer_backward(q, wo, wa, attn, gl, ga, ss, ls, outputs=grads,
                                                               workspace=pws, stream=stream),
        }
        ms = {k: time_launches(fn, stream, a.steps, a.warmup) for k, fn in fns.items()}
        fwd_peak = MFMA_BF16_PEAK_TFLOPS if dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
        el = 2 if dtype == "bf16" else 4
        # forward bytes: query features and both weight matrices read, reference
        # points read, locations and weights written (float32)
        fwd_bytes = (M * w["D"] * el + 3 * w["N_h"] * S * w["D"] * el + M * len(w["levels"]) * 2 * 4
                     + M * w["N_h"] * S * 3 * 4)
        line = {"producer": f"encoder shape, D={w['D']}, {dtype} inputs", "B": w["B"], "N_q": w["N_q"],
                "N_h": w["N_h"], "N_l": len(w["levels"]), "N_p": w["N_p"], "D": w["D"], "C_h": w["C_h"],
                "flop_forward": gemm_flop, "flop_backward": 2 * gemm_flop, "bytes_forward": fwd_bytes,
                "peak_tflops_forward": fwd_peak, "peak_tflops_backward": MFMA_F32_PEAK_TFLOPS,
                "peak_note": ("forward: bfloat16 matrix cores (operands as given, float32 accumulation); "
                              if dtype == "bf16" else "forward: float32 matrix cores; ")
                + "backward: float32 matrix cores (the gradients are float32)"}
        for k, flop, peak in (("forward", gemm_flop, fwd_peak), ("fused_forward", None, None),
                              ("backward", 2 * gemm_flop, MFMA_F32_PEAK_TFLOPS), ("sampler", None, None)):
            r = stats(ms[k])
            if flop:
                tf = flop / (r["ms_median"] * 1e-3) / 1e12
                r.update(tflops=tf, frac_of_peak=tf / peak)
            r["queries_per_s"] = M / (r["ms_median"] * 1e-3)
            line[k] = r
        f = line["forward"]
        f["hbm_gbs"] = fwd_bytes / (f["ms_median"] * 1e-3) / 1e9
        f["hbm_frac"] = f["hbm_gbs"] / HBM_PEAK_GBS
        f["bound"] = "mfma" if gemm_flop / (fwd_peak * 1e12) > fwd_bytes / (HBM_PEAK_GBS * 1e9) else "hbm"
        line["fused_forward"]["two_call_chain_ms"] = line["forward"]["ms_median"] + line["sampler"]["ms_median"]
        if not a.no_cpu_baseline:
            rows = 2048
            f64 = {k: p[k][:, :rows // w["B"]] for k in ("query", "reference_points")}
            t0 = time.perf_counter()
            reps = 0
            while time.perf_counter() - t0 < a.cpu_seconds / 4:
                l64, a64 = oprod.forward(f64["query"], f64["reference_points"], p["offset_weight"],
                                         p["offset_bias"], p["attention_weight"], p["attention_bias"],
                                         ss, w["N_h"], w["N_p"])
                oprod.backward(f64["query"], p["offset_weight"], p["attention_weight"], a64,
                               p["grad_sampling_locations"][:, :rows // w["B"]],
                               p["grad_attention_weights"][:, :rows // w["B"]], ss, w["N_h"], w["N_p"])
                reps += 1
            el = time.perf_counter() - t0
            line["cpu_oracle"] = {"queries_per_s": reps * rows / el, "kind": "oracle",
                                  "cores": len(os.sched_getaffinity(0)),
                                  "sample": f"{reps} forward+backward passes over {rows} rows "
                                            f"({el:.1f} s), float64 numpy (BLAS threads)"}
        print(json.dumps(line), flush=True)


# -------------------------------------------------------- mode variants ---

def mode_variants(a):
    """Forward and backward at workload 4's shapes (B=4, the square pyramid,
    N_q = L) with one mode changed at a time; one JSON line per case."""
    import torch
    from scale_deformable_attention_forward_amd import binding
    from scale_deformable_attention_forward_amd.workloads import WORKLOADS, make_inputs
    binding.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    wl = WORKLOADS[4]
    cases = (("as workload 4", "bf16", "BNLC", "B2QHLP", True, "border", (-0.05, 1.05)),
             ("zeros padding", "bf16", "BNLC", "B2QHLP", True, "zeros", (-0.05, 1.05)),
             ("border, locations U[0,1]", "bf16", "BNLC", "B2QHLP", True, "border", (0.0, 1.0)),
             ("fp32 value", "fp32", "BNLC", "B2QHLP", True, "border", (-0.05, 1.05)),
             ("BLNC/BQHLP2", "bf16", "BLNC", "BQHLP2", True, "border", (-0.05, 1.05)),
             ("align off", "bf16", "BNLC", "B2QHLP", False, "border", (-0.05, 1.05)),
             ("fp32 BLNC zeros align-off (workload 2 modes)", "fp32", "BLNC", "BQHLP2", False, "zeros",
              (-0.05, 1.05)))
    for name, dtype, vl, ll, align, pad, rng in cases:
        d = make_inputs(wl.B, wl.levels, wl.num_queries, wl.N_h, wl.C_h, wl.N_p, wl.seed, loc_range=rng,
                        value_dtype=dtype, value_layout=vl, sampling_locations_layout=ll, grad_seed=1004)
        d.update(align_corners=align, padding_mode=pad)
        t = _device_inputs(d, dev)
        fwd, bwd = _launchers(d, t, stream)
        fm = time_launches(fwd, stream, a.steps, a.warmup)
        bm = time_launches(bwd, stream, a.steps, a.warmup)
        q = wl.B * wl.num_queries
        print(json.dumps({"case": name, "fwd_ms": float(np.median(fm)), "bwd_ms": float(np.median(bm)),
                          "queries": q, "bwd_ns_per_query": float(np.median(bm)) * 1e6 / q}), flush=True)


# ----------------------------------------------------- generic backward ---

def generic_backward(a, d, t, stream):
    """Time msda_backward on its generic path (one channel per lane, float
    atomics into grad_value) at the same shape: a grad_value view 4 bytes off
    16-byte alignment rules out the tiled path. Prints one JSON line."""
    import torch
    from scale_deformable_attention_forward_amd import binding
    ss, ls = d["spatial_shapes"], d["level_start_index"]
    n = t["value"].numel()
    store = torch.empty(n + 1, dtype=t["value"].dtype, device=t["value"].device)
    gv = store[1:].view(t["value"].shape)
    gl, ga = torch.empty_like(t["loc"]), torch.empty_like(t["attn"])

    def bwd():
        binding.msda_backward(t["gout"], t["value"], ss, ls, t["loc"], t["attn"], grad_value=gv,
                              grad_sampling_locations=gl, grad_attention_weights=ga, stream=stream)
    ms = time_launches(bwd, stream, a.steps, a.warmup)
    bc = byte_counts(d)
    r = stats(ms)
    r.update({"path": "generic (float atomics)", "queries_per_s": bc["queries"] / (float(np.mean(ms)) * 1e-3),
              "gbs_counted": bc["backward"]["counted"] / (float(np.mean(ms)) * 1e-3) / 1e9,
              "global_atomic_lane_ops": 4 * bc["samples"] * d["value"].shape[-1],
              "counted_corner_updates": bc["counted_corners"]})
    print(json.dumps(r), flush=True)


# ------------------------------------------------------------------ main ---

def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {a.gpus} is not supported "
              "(the kernels shard by head with no communication, see the design notes)",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    if a.copy_calibration:
        # a plain copy of known size: reads and writes 1 GiB per launch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": src.numel() * 4, "launches": 5}), flush=True)
        return
    if a.report:
        report(a)
        return
    if a.producer:
        producer_report(a)
        return
    if a.mode_variants:
        mode_variants(a)
        return
    from scale_deformable_attention_forward_amd import binding
    from scale_deformable_attention_forward_amd.workloads import WORKLOADS, make_workload

    binding.load_library()   # raises if the HIP library is not built: no fallback
    wl = WORKLOADS[a.workload]
    d = make_workload(a.workload)
    if "grad_output" not in d:
        d["grad_output"] = make_workload(a.workload, grad_seed=1000 + a.workload)["grad_output"]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    t = _device_inputs(d, dev)
    fwd, bwd = _launchers(d, t, stream)
    if a.generic_backward:
        generic_backward(a, d, t, stream)
        return

    for _ in range(a.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    K = a.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        bwd()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f_ms = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)])
    b_ms = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)])
    span_ms = ev[0][0].elapsed_time(ev[K - 1][2])
    ms_per_step = span_ms / K

    cold, ceil = None, None
    if not a.quick:
        # cold caches: a 1 GiB scratch write before every launch (outside the events)
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cold = {"forward": stats(time_launches(fwd, stream, min(K, 30), 2, cold_buf=scratch)),
                "backward": stats(time_launches(bwd, stream, min(K, 30), 2, cold_buf=scratch)),
                "note": "30 launches each, a 1 GiB scratch write before every launch evicts L2 and the "
                        "256 MB last-level cache"}
        del scratch
        ceil = probe_ceilings(dev, stream)

    bc = byte_counts(d)
    comp = compulsory_bytes(d)
    Q = bc["queries"]
    t_fwd, t_bwd, per_kernel = measured_traffic() if a.workload == WORKLOAD_NUM else (None, None, {})
    traffic = {"forward": t_fwd, "backward": t_bwd}

    def kernel_line(name, ms):
        avg_s = float(np.mean(ms)) * 1e-3
        nominal, counted = bc[name]["nominal"], bc[name]["counted"]
        r = stats(ms)
        r.update({
            "queries_per_s": Q / avg_s,
            "bytes_nominal": nominal, "bytes_counted": counted,
            "gbs_nominal": nominal / avg_s / 1e9, "gbs_counted": counted / avg_s / 1e9,
            "l2_frac_counted": counted / avg_s / 1e9 / L2_PEAK_GBS,
            "effective_gbs_vs_hbm_peak": counted / avg_s / 1e9 / HBM_PEAK_GBS,
            "compulsory_bytes": comp[name],
        })
        tr = traffic[name]
        r["hbm_traffic_bytes"] = tr
        if tr is not None:
            r.update({"hbm_gbs": tr / avg_s / 1e9, "hbm_frac": tr / avg_s / 1e9 / HBM_PEAK_GBS,
                      "traffic_over_compulsory": tr / comp[name]})
        return r

    kf, kb = kernel_line("forward", f_ms), kernel_line("backward", b_ms)
    kf["launch"] = "forward_kernel (1 launch)"
    kb["launch"] = "msda_backward call: " + ", ".join(BACKWARD_KERNELS)
    dom_name, dom = ("backward", kb) if kb["ms_mean"] >= kf["ms_mean"] else ("forward", kf)
    roofline = {
        "bound": "l2", "kernel": dom_name, "launch": dom["launch"],
        "achieved": dom["gbs_counted"], "peak": L2_PEAK_GBS, "unit": "GB/s",
        "frac": dom["gbs_counted"] / L2_PEAK_GBS, "traffic": dom["hbm_traffic_bytes"],
        "bytes_per_launch": dom["bytes_counted"],
        "peak_derivation": f"{XCDS} XCDs x {L2_CHANNELS_PER_XCD} L2 channels x {L2_BYTES_PER_CLOCK} B/clock x "
                           f"{CLOCK_GHZ} GHz (L2 -> CU read path; the gathers hit L2 81-92% of the time)",
        "probe_measured_gbs": ceil,
        "frac_of_probe_l2_gather": None if ceil is None else dom["gbs_counted"] / ceil["l2_gather_128B_rows"],
        "forward_frac": kf["l2_frac_counted"],
        "hbm": {"traffic_bytes": dom["hbm_traffic_bytes"], "peak": HBM_PEAK_GBS,
                "achieved": dom.get("hbm_gbs"), "frac": dom.get("hbm_frac"),
                "compulsory_bytes": dom["compulsory_bytes"],
                "traffic_over_compulsory": dom.get("traffic_over_compulsory")},
        "note": "achieved = counted algorithmic bytes of one launch (corners in range with nonzero weight x "
                "C_h x 4 B, re-gather and scatter counted once each, plus every stream once) / its mean "
                "HIP-event time on the launch stream; traffic = memory-side bytes per launch from rocprofv3 "
                "FETCH_SIZE (x 2.0, what a 1 GiB copy gives; within 0.4% of 32 x TCC_EA0_RDREQ_DRAM_32B) "
                "and WRITE_SIZE (x 1.0 on the copy) (profiles/), null once a kernel source changed",
    }
    res = {
        "metric": METRIC,
        "value": Q / (ms_per_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.value_dtype == "bf16" else "f32",
        "data": "synthetic (seeded Deformable-DETR-shaped pyramid, no dataset)",
        "config": {"workload": f"{wl.name} forward+backward: B={wl.B}, levels={list(wl.levels)}, "
                               f"L={wl.L}, N_q={wl.num_queries}, N_h={wl.N_h}, C_h={wl.C_h}, N_l={wl.N_l}, "
                               f"N_p={wl.N_p}, {wl.value_dtype}, {wl.value_layout}/{wl.sampling_locations_layout}, "
                               f"{wl.padding_mode} padding, align_corners={wl.align_corners}",
                   "global_batch": wl.B, "queries_per_step": Q, "parallelism": "single GPU"},
        "roofline": roofline,
        "kernels": {"forward": kf, "backward": kb},
        "cold_caches": cold,
        "per_kernel_counters": per_kernel,
        "counted_corner_fraction": bc["counted_fraction"],
        "wall_s_timed": wall,
    }
    if not (a.no_cpu_baseline or a.quick):
        res["cpu_baseline"] = cpu_baseline(d, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
