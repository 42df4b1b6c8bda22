"""GPU: the forward and backward calls captured in a HIP graph (through
torch.cuda.CUDAGraph) and replayed. The library enqueues only kernels on the
caller's stream (it clears memory with kernels, never with a memset node) and
allocates nothing when every output and the workspace are passed in, so the
calls can be captured. Each replay gets new inputs copied into the captured
buffers, with eager work and synchronisation between replays, and must match
eager calls on the same inputs bitwise; eager results are checked against the
oracle once.
"""
import sys

import numpy as np
import pytest

from helpers import RTOL, compare, oracle_backward, oracle_forward, to_device, to_numpy
from scale_deformable_attention_forward_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype,C_h,levels,N_q", [
    ("fp32", 32, ((20, 30), (10, 15), (5, 8)), 500),   # halo-mode tile pass
    ("fp32", 32, ((60, 80), (8, 10)), 100),             # pixel mode (both levels)
    ("bf16", 32, ((20, 30), (10, 15)), 400),
    ("fp32", 6, ((12, 16), (6, 8)), 50),                # generic path (float atomics)
])
def test_graph_replays_match_eager(dtype, C_h, levels, N_q, gpu_device):
    import torch
    from scale_deformable_attention_forward_amd import binding
    _say(f"graph replay {dtype} C_h={C_h} levels={levels} N_q={N_q}")
    B, N_h, N_p = 2, 4, 4
    draws = [make_inputs(B, levels, N_q, N_h, C_h, N_p, seed, loc_range=(-0.05, 1.05), value_dtype=dtype,
                         grad_seed=seed + 100) for seed in (51, 52, 53)]
    ss, ls = draws[0]["spatial_shapes"], draws[0]["level_start_index"]
    mode = ("BLNC", "BQHLP2", False, "zeros")
    t0 = to_device(draws[0], gpu_device)
    # captured buffers: inputs, outputs and the workspace, all allocated before capture
    cap = {k: v.clone() for k, v in t0.items()}
    out = torch.empty((B, N_q, N_h * C_h), dtype=cap["value"].dtype, device=gpu_device)
    gv = torch.empty_like(cap["value"])
    gl = torch.empty_like(cap["sampling_locations"])
    ga = torch.empty_like(cap["attention_weights"])
    nws = binding.backward_workspace_bytes(cap["value"], ss, ls, cap["sampling_locations"], *mode)
    ws = torch.empty(max(1, nws), dtype=torch.uint8, device=gpu_device)

    def step():
        binding.msda_forward(cap["value"], ss, ls, cap["sampling_locations"], cap["attention_weights"], *mode,
                             output=out)
        binding.msda_backward(cap["grad_output"], cap["value"], ss, ls, cap["sampling_locations"],
                              cap["attention_weights"], *mode, grad_value=gv, grad_sampling_locations=gl,
                              grad_attention_weights=ga, workspace=ws)

    # warm up on a side stream, as torch asks before capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for i, d in enumerate(draws):
        t = to_device(d, gpu_device)
        for k in cap:
            cap[k].copy_(t[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in (out, gv, gl, ga)]
        # eager calls on the same inputs, into fresh outputs
        e_out = binding.msda_forward(t["value"], ss, ls, t["sampling_locations"], t["attention_weights"], *mode)
        e_gv, e_gl, e_ga = binding.msda_backward(t["grad_output"], t["value"], ss, ls, t["sampling_locations"],
                                                 t["attention_weights"], *mode)
        torch.cuda.synchronize()
        for name, a, b in zip(("output", "grad_value", "grad_loc", "grad_attn"), got, (e_out, e_gv, e_gl, e_ga)):
            if C_h % 4 != 0 and name == "grad_value":
                # the generic path sums with float atomics: equal up to summation order
                compare(f"replay {i} {name}", to_numpy(a), to_numpy(b), RTOL[dtype])
                continue
            assert torch.equal(a, b), f"replay {i}: {name} differs from the eager call"
        if i == 0:
            d.update(align_corners=False, padding_mode="zeros")
            compare("eager forward vs oracle", to_numpy(e_out), oracle_forward(d), RTOL[dtype])
            want = oracle_backward(d)
            for name, g, w in zip(("grad_value", "grad_loc", "grad_attn"), (e_gv, e_gl, e_ga), want):
                compare(f"eager {name} vs oracle", to_numpy(g), w, RTOL[dtype])
