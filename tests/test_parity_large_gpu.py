"""GPU parity for value tensors of 2^31 - 2^20 bytes and more.

Below that size the gathers read value through a raw buffer resource with
32-bit byte offsets; at and above it they take plain pointer loads of the
corners that carry weight ("MS Deformable Attention Kernel API Reference",
Parameters: value of shape (B, L, N_h, C_h) sets no size limit). These tests
run that pointer path against the CPU oracle: forward, backward (grad_A and
grad_loc from the pointer-path re-gather, grad_value from the tiled pass) and
the fused producer + sampler, on one 1024 x 2049 level with N_h * C_h = 256
(float32: 2.15 GB of value; bfloat16: a 1024 x 4097 level, 2.15 GB).

Sample locations are drawn U[0, 1] and a few are placed by hand where the
pointer path is most likely to go wrong: on the corner at element 2^29 (for
float32 that is 2^31 / 4, the buffer path's "no corner" offset) and on the
last rows and columns, whose byte offsets are past 2^31.
"""
import sys

import numpy as np
import pytest

from helpers import RTOL, oracle_backward, oracle_forward, to_numpy
from scale_deformable_attention_forward_amd.workloads import (bf16_bits_to_f32, bf16_round_bits, make_inputs,
                                                              make_large_value)

pytestmark = pytest.mark.gpu

N_H, C_H, N_P, N_Q = 8, 32, 4, 64
LEVEL = {"fp32": (1024, 2049), "bf16": (1024, 4097)}
# pixel coordinates (x, y) placed by hand (align_corners off, zeros padding)
TARGETS = [
    (1025.25, 1023.5),   # anchor (1025, 1023): pixel 2^21, element 2^29 of head 0 (fp32 level)
    (1024.5, 1022.75),   # its far corner is that pixel
    (2047.6, 1022.3),    # last column pair, last two rows
    (2048.4, 1022.6),    # right corners outside the level
    (1500.7, 1022.9),    # last row pair, mid-row
    (4095.3, 1022.2),    # bf16 level: last columns (outside the float32 level: zeros)
    (3073.25, 1023.5),   # bf16 level: anchor on pixel 2^22, element 2^30 of head 0 (2^31 / 2)
    (10.3, 0.2),
    (3.5, 500.5),
]


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _problem(dtype):
    H, W = LEVEL[dtype]
    # locations, weights and grad_output from the shared generator; the value
    # tensor from its float32 variant for tensors of gigabytes
    d = make_inputs(1, ((2, 2),), N_Q, N_H, C_H, N_P, seed=71, loc_range=(0.0, 1.0), grad_seed=72)
    d["spatial_shapes"] = ((H, W),)
    d["level_start_index"] = (0,)
    value, bits = make_large_value(1, H * W, N_H, C_H, seed=73, value_dtype=dtype)
    assert value.nbytes // (2 if dtype == "bf16" else 1) > (1 << 31) - (1 << 20)
    loc = d["sampling_locations"]
    k = 0
    for q in range(8):
        for h in range(N_H):
            for p in range(N_P):
                x, y = TARGETS[k % len(TARGETS)]
                k += 1
                loc[0, q, h, 0, p, 0] = (x + 0.5) / W
                loc[0, q, h, 0, p, 1] = (y + 0.5) / H
    d.update(value=value, value_dtype=dtype, align_corners=False, padding_mode="zeros")
    if bits is not None:
        d["value_bf16_bits"] = bits
        d["grad_output"] = bf16_bits_to_f32(bf16_round_bits(d["grad_output"]))
    return d


@pytest.fixture(scope="module", params=["fp32", "bf16"])
def large(request, gpu_device):
    import torch
    dtype = request.param
    _say(f"large value {dtype}: drawing inputs")
    d = _problem(dtype)
    dev = gpu_device
    t = {}
    if dtype == "bf16":
        t["value"] = torch.from_numpy(d["value_bf16_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
        t["grad_output"] = torch.from_numpy(d["grad_output"]).to(dev).to(torch.bfloat16)
    else:
        t["value"] = torch.from_numpy(d["value"]).to(dev)
        t["grad_output"] = torch.from_numpy(d["grad_output"]).to(dev)
    t["loc"] = torch.from_numpy(d["sampling_locations"]).to(dev)
    t["attn"] = torch.from_numpy(d["attention_weights"]).to(dev)
    yield d, t
    del t
    torch.cuda.empty_cache()


def _compare_sparse(name, got, want, rtol):
    """The comparison rule of helpers.compare, evaluated only where either side
    is nonzero (elsewhere both are 0 and the rule holds): grad_value here has
    half a billion elements and a few thousand nonzero ones."""
    got = np.asarray(got).reshape(-1)
    want = np.asarray(want).reshape(-1)
    assert got.shape == want.shape
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    rms = float(np.sqrt(np.mean(want * want)))
    nz = np.flatnonzero((want != 0) | (got != 0))
    assert nz.size > 0
    g, w = got[nz].astype(np.float64), want[nz].astype(np.float64)
    rel = np.abs(g - w) / (np.abs(w) + rms)
    i = int(np.argmax(rel))
    assert rel[i] <= rtol, f"{name}: max err {rel[i]:.3e} > {rtol:.1e} at element {nz[i]}: gpu {g[i]!r} oracle {w[i]!r}"


def _compare(name, got, want, rtol):
    from helpers import compare
    return compare(name, got, want, rtol)


def test_large_value_forward(large):
    import torch
    from scale_deformable_attention_forward_amd import msda_forward
    d, t = large
    _say(f"large value forward {d['value_dtype']}")
    out = msda_forward(t["value"], d["spatial_shapes"], d["level_start_index"], t["loc"], t["attn"])
    torch.cuda.synchronize()
    _compare(f"large forward {d['value_dtype']}", to_numpy(out), oracle_forward(d), RTOL[d["value_dtype"]])


def test_large_value_backward(large):
    import torch
    from scale_deformable_attention_forward_amd import msda_backward
    d, t = large
    _say(f"large value backward {d['value_dtype']}")
    gv, gl, ga = msda_backward(t["grad_output"], t["value"], d["spatial_shapes"], d["level_start_index"],
                               t["loc"], t["attn"])
    torch.cuda.synchronize()
    wgv, wgl, wga = oracle_backward(d)
    rtol = RTOL[d["value_dtype"]]
    _compare(f"large grad_attention_weights {d['value_dtype']}", to_numpy(ga), wga, rtol)
    _compare(f"large grad_sampling_locations {d['value_dtype']}", to_numpy(gl), wgl, rtol)
    got_gv = to_numpy(gv)
    del gv
    _compare_sparse(f"large grad_value {d['value_dtype']}", got_gv, wgv, rtol)
    # a sample reaches the element at the buffer path's "no corner" offset,
    # and samples reach elements past 2^31 bytes
    flat = wgv.reshape(-1)
    elem = 2 if d["value_dtype"] == "bf16" else 4
    assert flat[(1 << 31) // elem] != 0
    assert np.count_nonzero(flat[(1 << 31) // elem + 1:]) > 0


def test_large_value_fused_forward_equals_two_calls(large):
    """The fused producer + sampler takes the same pointer-path gather as the
    sampler: its output is bitwise that of msda_producer_forward followed by
    msda_forward (whose result the forward test holds to the oracle)."""
    import torch
    from scale_deformable_attention_forward_amd import binding
    from scale_deformable_attention_forward_amd.workloads import make_producer_inputs
    d, t = large
    if d["value_dtype"] != "fp32":
        pytest.skip("one dtype is enough for the fused gather's pointer path")
    _say("large value fused forward fp32")
    H, W = d["spatial_shapes"][0]
    p = make_producer_inputs(1, d["spatial_shapes"], N_Q, N_H, N_P, 32, seed=74)
    ref = p["reference_points"]
    for q in range(16):   # reference points on the hand-placed targets (offsets are about 2 pixels)
        x, y = TARGETS[q % len(TARGETS)]
        ref[0, q, 0] = ((x + 0.5) / W, (y + 0.5) / H)
    dev = t["value"].device
    q, r, wo, bo, wa, ba = (torch.from_numpy(np.ascontiguousarray(p[k])).to(dev) for k in
                            ("query", "reference_points", "offset_weight", "offset_bias", "attention_weight",
                             "attention_bias"))
    ss, ls = d["spatial_shapes"], d["level_start_index"]
    loc, attn = binding.msda_producer_forward(q, r, wo, bo, wa, ba, ss, ls, N_H)
    two = binding.msda_forward(t["value"], ss, ls, loc, attn)
    fused = binding.msda_fused_forward(t["value"], ss, ls, q, r, wo, bo, wa, ba)
    torch.cuda.synchronize()
    assert torch.equal(fused, two)
    assert float(two.abs().max()) > 0
