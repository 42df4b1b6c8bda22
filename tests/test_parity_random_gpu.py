"""GPU parity on seeded random problems: level counts and sizes (rows or
columns of one pixel included), batch, heads, channels (multiples of 4 up to
64 take the fast paths, the others the generic ones), points, query counts,
both value dtypes, layouts, padding modes and align_corners, with locations
spread over and beyond the levels or clustered onto a few pixels. Each case
compares the forward output and all three gradients with the oracle under
the comparison rule in helpers.py, grad_value with the magnitude of its
terms in the scale (a 1x1 level takes every sample of its level on one
pixel).
"""
import sys

import numpy as np
import pytest

from helpers import RTOL, compare, oracle_backward, oracle_forward, to_device, to_numpy
from scale_deformable_attention_forward_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu

N_CASES = 200


def _case(i):
    r = np.random.default_rng(7000 + i)
    n_l = int(r.integers(1, 6))
    levels = []
    for _ in range(n_l):
        h, w = int(r.integers(1, 71)), int(r.integers(1, 71))
        if r.random() < 0.15:
            h = 1
        if r.random() < 0.15:
            w = 1
        levels.append((h, w))
    c_h = int(r.choice([4, 8, 12, 16, 20, 32, 48, 64, 6, 10]))
    case = dict(levels=tuple(levels), B=int(r.integers(1, 4)), N_h=int(r.integers(1, 5)), C_h=c_h,
                N_p=int(r.integers(1, 7)), N_q=int(np.exp(r.uniform(0.0, np.log(3000.0)))),
                dtype="bf16" if r.random() < 0.3 else "fp32",
                value_layout=str(r.choice(["BLNC", "BNLC"])), loc_layout=str(r.choice(["BQHLP2", "B2QHLP"])),
                align=bool(r.random() < 0.5), pad=str(r.choice(["zeros", "border"])),
                dist=str(r.choice(["uniform", "clustered"])), seed=7000 + i)
    # keep every case small enough for the oracle
    while case["B"] * case["N_q"] * case["N_h"] * n_l * case["N_p"] * case["C_h"] > 2_000_000:
        case["N_q"] = max(1, case["N_q"] // 2)
    return case


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_problem(i, gpu_device):
    from scale_deformable_attention_forward_amd import msda_backward, msda_forward
    import torch
    c = _case(i)
    print(f"[case] random {i}: {c}", flush=True)
    sys.stdout.flush()
    d = make_inputs(c["B"], c["levels"], c["N_q"], c["N_h"], c["C_h"], c["N_p"], c["seed"],
                    loc_dist=c["dist"], loc_range=(-0.2, 1.2), value_dtype=c["dtype"],
                    value_layout=c["value_layout"], sampling_locations_layout=c["loc_layout"],
                    grad_seed=c["seed"] + 1)
    d.update(align_corners=c["align"], padding_mode=c["pad"])
    t = to_device(d, gpu_device)
    args = (d["spatial_shapes"], d["level_start_index"], t["sampling_locations"], t["attention_weights"],
            d["value_layout"], d["sampling_locations_layout"], d["align_corners"], d["padding_mode"])
    out = msda_forward(t["value"], *args)
    grads = msda_backward(t["grad_output"], t["value"], *args)
    torch.cuda.synchronize()
    rtol = RTOL[c["dtype"]]
    compare(f"forward {i}", to_numpy(out), oracle_forward(d), rtol)
    want = oracle_backward(d)
    # 1x1 levels and clustered locations pile hundreds to thousands of
    # samples onto one pixel, whose grad_value is then a sum of that many
    # cancelling terms: it is judged against their magnitude too
    mag = oracle_backward(d, grad_output=np.abs(d["grad_output"]), attention_weights=np.abs(d["attention_weights"]),
                          compute_grad_sampling_locations=False, compute_grad_attention_weights=False)[0]
    compare(f"grad_value {i}", to_numpy(grads[0]), want[0], rtol, magnitude=mag)
    for name, got, w in zip(("grad_sampling_locations", "grad_attention_weights"), grads[1:], want[1:]):
        compare(f"{name} {i}", to_numpy(got), w, rtol)


N_MANY_RUN_CASES = 100


def _many_run_case(i):
    """Narrow but long problems: more than 2,048 samples per (b, h, level), so
    the bucketing takes several runs (count, scan and fill kernels) and dense
    levels take several passes or split bands."""
    r = np.random.default_rng(9000 + i)
    n_l = int(r.integers(1, 4))
    levels = tuple((int(r.integers(1, 71)), int(r.integers(1, 71))) for _ in range(n_l))
    return dict(levels=levels, B=int(r.integers(1, 3)), N_h=int(r.integers(1, 3)), C_h=int(r.choice([4, 8])),
                N_p=int(r.integers(2, 5)), N_q=int(r.integers(1000, 20001)),
                dtype="bf16" if r.random() < 0.3 else "fp32",
                value_layout=str(r.choice(["BLNC", "BNLC"])), loc_layout=str(r.choice(["BQHLP2", "B2QHLP"])),
                align=bool(r.random() < 0.5), pad=str(r.choice(["zeros", "border"])),
                dist=str(r.choice(["uniform", "clustered"])), seed=9000 + i)


@pytest.mark.parametrize("i", range(N_MANY_RUN_CASES))
def test_random_problem_many_runs(i, gpu_device):
    from scale_deformable_attention_forward_amd import msda_backward
    import torch
    c = _many_run_case(i)
    print(f"[case] random many-run {i}: {c}", flush=True)
    sys.stdout.flush()
    d = make_inputs(c["B"], c["levels"], c["N_q"], c["N_h"], c["C_h"], c["N_p"], c["seed"],
                    loc_dist=c["dist"], loc_range=(-0.2, 1.2), value_dtype=c["dtype"],
                    value_layout=c["value_layout"], sampling_locations_layout=c["loc_layout"],
                    grad_seed=c["seed"] + 1)
    d.update(align_corners=c["align"], padding_mode=c["pad"])
    t = to_device(d, gpu_device)
    args = (d["spatial_shapes"], d["level_start_index"], t["sampling_locations"], t["attention_weights"],
            d["value_layout"], d["sampling_locations_layout"], d["align_corners"], d["padding_mode"])
    grads = msda_backward(t["grad_output"], t["value"], *args)
    torch.cuda.synchronize()
    rtol = RTOL[c["dtype"]]
    want = oracle_backward(d)
    mag = oracle_backward(d, grad_output=np.abs(d["grad_output"]), attention_weights=np.abs(d["attention_weights"]),
                          compute_grad_sampling_locations=False, compute_grad_attention_weights=False)[0]
    compare(f"grad_value many-run {i}", to_numpy(grads[0]), want[0], rtol, magnitude=mag)
    for name, got, w in zip(("grad_sampling_locations", "grad_attention_weights"), grads[1:], want[1:]):
        compare(f"{name} many-run {i}", to_numpy(got), w, rtol)
