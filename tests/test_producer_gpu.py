"""GPU parity of the producer of sampling locations and attention weights
(msda_producer_forward, msda_fused_forward, msda_producer_backward) through
the C ABI, against the CPU oracle (oracle/producer.py, and oracle.forward for
the sampler half of the fused kernel) on the same seeded inputs.

Tolerances. The producer's outputs are float32 results of float32 (or exact
bfloat16) inputs, so they are held to the float32 rule of helpers.py
(rtol 1e-5 against |oracle| + rms) for both input dtypes; a bfloat16
grad_query is rounded once to bfloat16 and takes the bfloat16 rule.

The fused kernel is checked three ways: (a) bitwise against the two-call
chain producer -> sampler on the GPU (it computes the same float32 values by
construction); (b) against the oracle chain to the float32 rule on dyadic
inputs, where the projection and the normalisation are exact in float32 so
both sides sample at the same locations; (c) at the encoder shape with
normal inputs, against the oracle chain within a bound derived from the
arithmetic: a location differs from the oracle's float32 rounding of it by
at most 2^-22 (two units in the last place below 2), which moves the pixel
coordinate by (W or H) * 2^-22 and the sample by at most 2 * max|value| per
pixel of movement, weighted by the attention weights (summing to 1).
"""
import sys

import numpy as np
import pytest

import oracle
from oracle import producer as oracle_producer
from helpers import RTOL, compare
from scale_deformable_attention_forward_amd.workloads import (ENCODER_LEVELS, make_inputs,
                                                              make_producer_inputs)

pytestmark = pytest.mark.gpu

ENCODER = dict(B=2, levels=ENCODER_LEVELS, N_q=22223, N_h=8, N_p=4, D=256)


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _t(a, dev, bf16_bits=None):
    import torch
    if bf16_bits is not None:
        return torch.from_numpy(bf16_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def _dev_inputs(p, dev, bias=True):
    bf = p["value_dtype"] == "bf16"
    out = {k: _t(p[k], dev, p.get(k + "_bf16_bits") if bf else None)
           for k in ("query", "offset_weight", "attention_weight")}
    out["reference_points"] = _t(p["reference_points"], dev)
    out["offset_bias"] = _t(p["offset_bias"], dev) if bias else None
    out["attention_bias"] = _t(p["attention_bias"], dev) if bias else None
    return out


def _oracle_forward(p, layout="BQHLP2", bias=True):
    return oracle_producer.forward(p["query"], p["reference_points"], p["offset_weight"],
                                   p["offset_bias"] if bias else None, p["attention_weight"],
                                   p["attention_bias"] if bias else None, p["spatial_shapes"], p["N_h"],
                                   p["N_p"], layout)


def _gpu_producer(p, dev, layout="BQHLP2", bias=True):
    import torch
    from scale_deformable_attention_forward_amd import msda_producer_forward
    t = _dev_inputs(p, dev, bias)
    loc, attn = msda_producer_forward(t["query"], t["reference_points"], t["offset_weight"], t["offset_bias"],
                                      t["attention_weight"], t["attention_bias"], p["spatial_shapes"],
                                      p["level_start_index"], p["N_h"], layout)
    torch.cuda.synchronize()
    return loc, attn


def _check_producer(p, dev, tag, layout="BQHLP2", bias=True):
    _say(f"producer forward {tag}")
    loc, attn = _gpu_producer(p, dev, layout, bias)
    wl, wa = _oracle_forward(p, layout, bias)
    compare(f"sampling_locations {tag}", _np(loc), wl, RTOL["fp32"])
    compare(f"attention_weights {tag}", _np(attn), wa, RTOL["fp32"])


# ------------------------------------------------------------- forward ---

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_producer_forward_encoder_shape(dtype, gpu_device):
    p = make_producer_inputs(**ENCODER, seed=21, value_dtype=dtype)
    _check_producer(p, gpu_device, f"encoder D=256 {dtype}")


@pytest.mark.parametrize("layout", ["BQHLP2", "B2QHLP"])
@pytest.mark.parametrize("levels,N_q,N_h,N_p,D", [
    (((7, 9), (4, 5), (1, 1)), 37, 3, 3, 37),        # S = 9 (not a power of two), D % 4 != 0, ragged rows
    (((6, 5),), 65, 2, 1, 8),                         # S = 1, one row past a tile
    (((8, 8), (4, 4), (2, 2), (1, 1)), 130, 2, 16, 40),  # S = 64: 12 column tiles
    (((5, 11), (3, 2)), 64, 5, 2, 300),               # D past one staging step, not a multiple of 32
])
def test_producer_forward_shapes(layout, levels, N_q, N_h, N_p, D, gpu_device):
    p = make_producer_inputs(2, levels, N_q, N_h, N_p, D, seed=22)
    _check_producer(p, gpu_device, f"levels={levels} N_q={N_q} N_h={N_h} N_p={N_p} D={D} {layout}", layout)


def test_producer_forward_without_biases(gpu_device):
    p = make_producer_inputs(1, ((9, 7), (3, 3)), 50, 4, 2, 24, seed=23)
    _check_producer(p, gpu_device, "no biases", bias=False)


def test_producer_forward_bf16_ragged(gpu_device):
    p = make_producer_inputs(3, ((7, 9), (4, 5)), 29, 2, 4, 20, seed=24, value_dtype="bf16")
    _check_producer(p, gpu_device, "bf16 ragged", "B2QHLP")


def test_producer_forward_is_bitwise_stable(gpu_device):
    p = make_producer_inputs(1, ENCODER_LEVELS, 3000, 8, 4, 256, seed=25)
    a = _gpu_producer(p, gpu_device)
    b = _gpu_producer(p, gpu_device)
    for x, y in zip(a, b):
        assert (x.cpu().numpy().view(np.uint32) == y.cpu().numpy().view(np.uint32)).all()


# --------------------------------------------------------------- fused ---

def _value_for(p, C_h, value_dtype="fp32", value_layout="BLNC", seed=31):
    B, N_q = p["query"].shape[:2]
    return make_inputs(B, p["spatial_shapes"], N_q, p["N_h"], C_h, p["N_p"], seed, value_dtype=value_dtype,
                       value_layout=value_layout)


def _gpu_fused(p, v, dev, mode):
    import torch
    from scale_deformable_attention_forward_amd import msda_fused_forward
    t = _dev_inputs(p, dev)
    bf = v["value_dtype"] == "bf16"
    val = _t(v["value"], dev, v["value_bf16_bits"] if bf else None)
    res = msda_fused_forward(val, p["spatial_shapes"], p["level_start_index"], t["query"], t["reference_points"],
                             t["offset_weight"], t["offset_bias"], t["attention_weight"], t["attention_bias"],
                             *mode, return_sampling=True)
    torch.cuda.synchronize()
    return res, val


def _gpu_chain(p, val, dev, mode):
    import torch
    from scale_deformable_attention_forward_amd import msda_forward
    loc, attn = _gpu_producer(p, dev, mode[1])
    out = msda_forward(val, p["spatial_shapes"], p["level_start_index"], loc, attn, *mode)
    torch.cuda.synchronize()
    return out, loc, attn


def _bits(t):
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.cpu().numpy().view(np.uint32)


MODES = [("BLNC", "BQHLP2", False, "zeros"), ("BNLC", "B2QHLP", True, "border"),
         ("BLNC", "B2QHLP", False, "border"), ("BNLC", "BQHLP2", True, "zeros")]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fused_equals_producer_then_sampler_encoder_shape(dtype, gpu_device):
    p = make_producer_inputs(**ENCODER, seed=32, value_dtype=dtype)
    v = _value_for(p, 32, dtype)
    mode = MODES[0]
    _say(f"fused vs chain encoder {dtype}")
    (out, loc, attn), val = _gpu_fused(p, v, gpu_device, mode)
    c_out, c_loc, c_attn = _gpu_chain(p, val, gpu_device, mode)
    for name, a, b in (("output", out, c_out), ("loc", loc, c_loc), ("attn", attn, c_attn)):
        diff = int((_bits(a) != _bits(b)).sum())
        assert diff == 0, f"{name}: {diff} elements differ from the two-call chain"


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("C_h", [32, 6])
def test_fused_equals_chain_modes(mode, C_h, gpu_device):
    p = make_producer_inputs(2, ((7, 9), (4, 5), (2, 3)), 70, 3, 3, 20, seed=33)
    v = _value_for(p, C_h, value_layout=mode[0])
    _say(f"fused vs chain {mode} C_h={C_h}")
    (out, loc, attn), val = _gpu_fused(p, v, gpu_device, mode)
    c_out, c_loc, c_attn = _gpu_chain(p, val, gpu_device, mode)
    for name, a, b in (("output", out, c_out), ("loc", loc, c_loc), ("attn", attn, c_attn)):
        assert (_bits(a) == _bits(b)).all(), name


@pytest.mark.parametrize("mode", MODES)
def test_fused_matches_oracle_on_exact_locations(mode, gpu_device):
    levels = ((16, 16), (8, 8), (4, 4), (2, 2))
    p = make_producer_inputs(2, levels, 300, 4, 4, 64, seed=34, dyadic=True)
    v = _value_for(p, 32, value_layout=mode[0])
    _say(f"fused vs oracle, dyadic inputs {mode}")
    (out, loc, attn), _ = _gpu_fused(p, v, gpu_device, mode)
    wl, wa = _oracle_forward(p, mode[1])
    assert (_np(loc) == wl).all(), "exact locations differ"
    compare("attention_weights dyadic", _np(attn), wa, RTOL["fp32"])
    want = oracle.forward(v["value"], p["spatial_shapes"], p["level_start_index"], wl.astype(np.float32), wa,
                          *mode)
    compare(f"fused output dyadic {mode}", _np(out), want, RTOL["fp32"])


def test_fused_matches_oracle_within_location_bound_encoder_shape(gpu_device):
    p = make_producer_inputs(**ENCODER, seed=35)
    v = _value_for(p, 32)
    mode = MODES[0]
    _say("fused vs oracle encoder, derived location bound")
    (out, loc, attn), _ = _gpu_fused(p, v, gpu_device, mode)
    wl, wa = _oracle_forward(p)
    compare("sampling_locations (fused)", _np(loc), wl, RTOL["fp32"])
    want = oracle.forward(v["value"], p["spatial_shapes"], p["level_start_index"], wl.astype(np.float32), wa,
                          *mode)
    got = _np(out)
    rms = float(np.sqrt(np.mean(want * want)))
    H0, W0 = p["spatial_shapes"][0]
    bound = RTOL["fp32"] * (np.abs(want) + rms) + 2.0 * float(np.abs(v["value"]).max()) * (W0 + H0) * 2.0 ** -22
    err = np.abs(got - want)
    assert (err <= bound).all(), f"max excess {(err - bound).max():.3e}"
    # the bound is loose; most elements are much closer
    assert np.median(err / (np.abs(want) + rms)) < 1e-5


def test_fused_without_sampling_outputs(gpu_device):
    import torch
    from scale_deformable_attention_forward_amd import msda_fused_forward
    p = make_producer_inputs(1, ((9, 7), (3, 3)), 100, 2, 4, 32, seed=36)
    v = _value_for(p, 16)
    t = _dev_inputs(p, gpu_device)
    val = _t(v["value"], gpu_device)
    args = (val, p["spatial_shapes"], p["level_start_index"], t["query"], t["reference_points"],
            t["offset_weight"], t["offset_bias"], t["attention_weight"], t["attention_bias"])
    a = msda_fused_forward(*args)
    b, _, _ = msda_fused_forward(*args, return_sampling=True)
    torch.cuda.synchronize()
    assert (_bits(a) == _bits(b)).all()


# ------------------------------------------------------------ backward ---

def _gpu_producer_backward(p, dev, layout="BQHLP2", compute=None, grads=(True, True)):
    import torch
    from scale_deformable_attention_forward_amd import msda_producer_backward
    from scale_deformable_attention_forward_amd.binding import PRODUCER_GRADS
    t = _dev_inputs(p, dev)
    _, attn = _oracle_forward(p, layout)
    gl = p["grad_sampling_locations"]
    if layout == "B2QHLP":
        gl = np.ascontiguousarray(np.moveaxis(gl, -1, 1))
    A = _t(attn.astype(np.float32), dev)
    gl_t = _t(gl, dev) if grads[0] else None
    ga_t = _t(p["grad_attention_weights"], dev) if grads[1] else None
    out = msda_producer_backward(t["query"], t["offset_weight"], t["attention_weight"], A, gl_t, ga_t,
                                 p["spatial_shapes"], p["level_start_index"], layout,
                                 compute=PRODUCER_GRADS if compute is None else compute)
    torch.cuda.synchronize()
    return out, attn.astype(np.float32), gl


def _oracle_backward(p, attn, gl, layout, grads=(True, True)):
    z = np.zeros_like
    return oracle_producer.backward(p["query"], p["offset_weight"], p["attention_weight"], attn,
                                    gl if grads[0] else z(gl), p["grad_attention_weights"] if grads[1]
                                    else z(p["grad_attention_weights"]), p["spatial_shapes"], p["N_h"],
                                    p["N_p"], layout)


def _check_backward(p, dev, tag, layout="BQHLP2", grads=(True, True)):
    _say(f"producer backward {tag}")
    got, attn, gl = _gpu_producer_backward(p, dev, layout, grads=grads)
    want = _oracle_backward(p, attn, gl, layout, grads)
    for k, w in want.items():
        rt = RTOL["bf16"] if (k == "query" and p["value_dtype"] == "bf16") else RTOL["fp32"]
        compare(f"grad {k} {tag}", _np(got[k]), w, rt)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_producer_backward_encoder_shape(dtype, gpu_device):
    p = make_producer_inputs(**ENCODER, seed=41, value_dtype=dtype, grad_seed=42)
    _check_backward(p, gpu_device, f"encoder D=256 {dtype}")


@pytest.mark.parametrize("layout", ["BQHLP2", "B2QHLP"])
@pytest.mark.parametrize("levels,N_q,N_h,N_p,D", [
    (((7, 9), (4, 5), (1, 1)), 37, 3, 3, 37),
    (((6, 5),), 65, 2, 1, 8),
    (((8, 8), (4, 4), (2, 2), (1, 1)), 130, 2, 16, 40),
    (((5, 11), (3, 2)), 64, 5, 2, 300),
])
def test_producer_backward_shapes(layout, levels, N_q, N_h, N_p, D, gpu_device):
    p = make_producer_inputs(2, levels, N_q, N_h, N_p, D, seed=43, grad_seed=44)
    _check_backward(p, gpu_device, f"levels={levels} N_q={N_q} N_h={N_h} N_p={N_p} D={D} {layout}", layout)


@pytest.mark.parametrize("grads", [(True, False), (False, True)])
def test_producer_backward_one_output_gradient(grads, gpu_device):
    p = make_producer_inputs(2, ((7, 9), (4, 5)), 90, 4, 2, 48, seed=45, grad_seed=46)
    _check_backward(p, gpu_device, f"grads={grads}", grads=grads)


@pytest.mark.parametrize("compute", [("query",), ("reference_points",), ("offset_weight", "attention_bias"),
                                     ("attention_weight", "offset_bias", "reference_points")])
def test_producer_backward_selected_gradients(compute, gpu_device):
    p = make_producer_inputs(2, ((7, 9), (4, 5)), 90, 4, 2, 48, seed=47, grad_seed=48)
    _say(f"producer backward compute={compute}")
    got, attn, gl = _gpu_producer_backward(p, gpu_device, compute=compute)
    want = _oracle_backward(p, attn, gl, "BQHLP2")
    for k in want:
        if k in compute:
            compare(f"grad {k}", _np(got[k]), want[k], RTOL["fp32"])
        else:
            assert got[k] is None


def test_producer_backward_is_bitwise_stable(gpu_device):
    p = make_producer_inputs(2, ENCODER_LEVELS, 2000, 8, 4, 256, seed=49, grad_seed=50)
    a, _, _ = _gpu_producer_backward(p, gpu_device)
    b, _, _ = _gpu_producer_backward(p, gpu_device)
    for k in a:
        assert (_bits(a[k]) == _bits(b[k])).all(), k


def test_producer_backward_empty_rows_zero_weight_grads(gpu_device):
    import torch
    from scale_deformable_attention_forward_amd import msda_producer_backward
    p = make_producer_inputs(2, ((7, 9), (4, 5)), 0, 2, 2, 16, seed=51, grad_seed=52)
    t = _dev_inputs(p, gpu_device)
    A = torch.zeros((2, 0, 2, 2, 2), dtype=torch.float32, device=gpu_device)
    out = msda_producer_backward(t["query"], t["offset_weight"], t["attention_weight"], A, None, None,
                                 p["spatial_shapes"], p["level_start_index"])
    torch.cuda.synchronize()
    for k in ("offset_weight", "offset_bias", "attention_weight", "attention_bias"):
        assert out[k] is not None and (out[k] == 0).all(), k


def test_producer_autograd_matches_oracle(gpu_device):
    import torch
    from scale_deformable_attention_forward_amd import MSDAProducer
    p = make_producer_inputs(2, ((7, 9), (4, 5)), 45, 3, 2, 24, seed=53, grad_seed=54)
    t = _dev_inputs(p, gpu_device)
    leaves = {k: t[k].clone().requires_grad_(True) for k in ("query", "reference_points", "offset_weight",
                                                             "offset_bias", "attention_weight",
                                                             "attention_bias")}
    loc, attn = MSDAProducer.apply(leaves["query"], leaves["reference_points"], leaves["offset_weight"],
                                   leaves["offset_bias"], leaves["attention_weight"], leaves["attention_bias"],
                                   p["spatial_shapes"], p["level_start_index"], p["N_h"])
    gl = _t(p["grad_sampling_locations"], gpu_device)
    ga = _t(p["grad_attention_weights"], gpu_device)
    ((loc * gl).sum() + (attn * ga).sum()).backward()
    _, wa = _oracle_forward(p)
    want = _oracle_backward(p, wa.astype(np.float32), p["grad_sampling_locations"], "BQHLP2")
    for k, w in want.items():
        compare(f"autograd grad {k}", _np(leaves[k].grad), w, RTOL["fp32"])
