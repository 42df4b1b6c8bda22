"""Benchmark of the multi-scale deformable attention hot path on one MI355X.

One step = one forward (msda_forward) plus one backward (msda_backward, all
three gradients) over the encoder-shaped workload: B=2, four levels
(100,167),(50,84),(25,42),(13,21) so L = N_q = 22223, N_h=8, C_h=32, N_p=4,
float32, BLNC / BQHLP2, zeros padding, align_corners off; locations
U[-0.05, 1.05], softmax attention weights, grad_output ~ N(0, 1). Inputs are
seeded, synthetic, and resident in HBM before the timed region starts.

Prints ONE JSON line. `value` is queries/s of whole steps; `roofline` is the
dominant launch's algorithmic bytes over its average duration (HIP events on
the stream the kernels run on) against the 8 TB/s HBM peak; `cpu_baseline` is
the CPU oracle timed on a bounded sample of the same workload on this host.

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
    ap.add_argument("--cold", action="store_true",
                    help="also time steps with a 1 GiB scratch write before each launch (caches cold)")
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
    """HBM bytes per forward launch and per backward call, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary scaled by its copy calibration
    (per-dispatch bytes times dispatches per call), plus the L2 hit rate of each
    kernel; (None, None, {}) when a kernel source changed since the counters
    were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None, None, {}
    for rel, digest in rec["sources_sha256"].items():
        path = os.path.join(ROOT, rel)
        if not os.path.exists(path) or hashlib.sha256(open(path, "rb").read()).hexdigest() != digest:
            return None, None, {}
    ff = rec["copy_calibration"]["fetch_factor"]
    wf = rec["copy_calibration"]["write_factor"]
    fwd = bwd = 0.0
    per = {}
    for name, c in rec["per_dispatch"].items():
        b = (c["FETCH_SIZE_KiB"] * ff + c["WRITE_SIZE_KiB"] * wf) * 1024.0 * c["dispatches_per_call"]
        per[name] = {"hbm_bytes_per_call": b, "l2_hit_pct": c.get("L2_hit_pct")}
        if name.startswith("forward_kernel"):
            fwd += b
        else:
            bwd += b
    return fwd, bwd, per


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
    return {"ms_mean": float(np.mean(ms)), "ms_median": float(np.median(ms)),
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
    """The CPU oracle on the same inputs: whole forward+backward steps,
    repeated until about target_s seconds have run."""
    import oracle
    args = (d["spatial_shapes"], d["level_start_index"])
    B, N_q = d["attention_weights"].shape[:2]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(d["value"], *args, d["sampling_locations"], d["attention_weights"])
        oracle.backward(d["grad_output"], d["value"], *args, d["sampling_locations"],
                        d["attention_weights"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 50:
            break
    return {"value": reps * B * N_q / el, "unit": "queries/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{reps} full forward+backward step(s) of the same workload ({reps * B * N_q} "
                      f"queries, {el:.1f} s), fp64 C oracle with OpenMP"}


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
                "frac_of_hbm_peak_counted": bc[name]["counted"] / avg_s / 1e9 / HBM_PEAK_GBS,
            }
        if not a.no_cpu_baseline:
            for name in ("forward", "backward"):
                tgt = a.cpu_seconds / 4
                qa, ca, sa = oracle_rate(d, (name,), tgt)
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
    FLOP/s against the float32 matrix-core peak, and the CPU oracle (float64
    numpy) on a bounded slice of rows."""
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
        line = {"producer": f"encoder shape, D={w['D']}, {dtype} inputs", "B": w["B"], "N_q": w["N_q"],
                "N_h": w["N_h"], "N_l": len(w["levels"]), "N_p": w["N_p"], "D": w["D"], "C_h": w["C_h"],
                "flop_forward": gemm_flop, "flop_backward": 2 * gemm_flop,
                "peak_tflops": MFMA_F32_PEAK_TFLOPS, "peak_note": "float32 matrix cores (bfloat16 inputs are "
                                                                  "widened exactly and multiplied in float32)"}
        for k, flop in (("forward", gemm_flop), ("fused_forward", None), ("backward", 2 * gemm_flop),
                        ("sampler", None)):
            r = stats(ms[k])
            if flop:
                tf = flop / (r["ms_mean"] * 1e-3) / 1e12
                r.update(tflops=tf, frac_of_peak=tf / MFMA_F32_PEAK_TFLOPS)
            r["queries_per_s"] = M / (r["ms_mean"] * 1e-3)
            line[k] = r
        line["fused_forward"]["two_call_chain_ms"] = line["forward"]["ms_mean"] + line["sampler"]["ms_mean"]
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
    from scale_deformable_attention_forward_amd import binding
    from scale_deformable_attention_forward_amd.workloads import WORKLOADS, make_workload

    binding.load_library()   # raises if the HIP library is not built: no fallback
    wl = WORKLOADS[WORKLOAD_NUM]
    d = make_workload(WORKLOAD_NUM)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    t = _device_inputs(d, dev)
    fwd, bwd = _launchers(d, t, stream)

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

    cold = None
    if a.cold:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        cold = {"forward": stats(time_launches(fwd, stream, min(K, 30), 2, cold_buf=scratch)),
                "backward": stats(time_launches(bwd, stream, min(K, 30), 2, cold_buf=scratch))}
        del scratch

    bc = byte_counts(d)
    Q = bc["queries"]

    def kernel_line(name, ms):
        avg_s = float(np.mean(ms)) * 1e-3
        nominal = bc[name]["nominal"]
        counted = bc[name]["counted"]
        r = stats(ms)
        r.update({
            "queries_per_s": Q / avg_s,
            "bytes_nominal": nominal, "bytes_counted": counted,
            "gbs_nominal": nominal / avg_s / 1e9, "gbs_counted": counted / avg_s / 1e9,
            "frac_counted": counted / avg_s / 1e9 / HBM_PEAK_GBS,
        })
        return r

    kf, kb = kernel_line("forward", f_ms), kernel_line("backward", b_ms)
    t_fwd, t_bwd, per_kernel = measured_traffic()
    kf["traffic"], kb["traffic"] = t_fwd, t_bwd
    kf["launch"] = "forward_kernel (1 launch)"
    kb["launch"] = "msda_backward call: " + ", ".join(BACKWARD_KERNELS)
    dom_name, dom = ("backward", kb) if kb["ms_mean"] >= kf["ms_mean"] else ("forward", kf)
    achieved = dom["bytes_nominal"] / (dom["ms_mean"] * 1e-3) / 1e9
    roofline = {
        "bound": "hbm", "kernel": dom_name, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": achieved / HBM_PEAK_GBS, "traffic": dom["traffic"],
        "bytes_per_launch": dom["bytes_nominal"],
        "launch": dom["launch"],
        "note": "achieved = algorithmic bytes (nominal per-query figure x queries, 4 corners per sample) "
                "/ mean HIP-event time of one launch; achieved_counted uses the corners the method must "
                "read; traffic = HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE (profiles/)",
        "achieved_counted": dom["gbs_counted"],
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
        "dtype": "f32",
        "data": "synthetic (seeded Deformable-DETR-shaped pyramid, no dataset)",
        "config": {"workload": f"{wl.name} forward+backward: B={wl.B}, levels={list(wl.levels)}, "
                               f"L=N_q={wl.L}, N_h={wl.N_h}, C_h={wl.C_h}, N_l={wl.N_l}, N_p={wl.N_p}, "
                               "BLNC/BQHLP2, zeros padding, align_corners=False",
                   "global_batch": wl.B, "queries_per_step": Q, "parallelism": "single GPU"},
        "roofline": roofline,
        "kernels": {"forward": kf, "backward": kb},
        "per_kernel_counters": per_kernel,
        "counted_corner_fraction": bc["counted_fraction"],
        "wall_s_timed": wall,
    }
    if cold is not None:
        res["cold_caches"] = cold
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(d, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
