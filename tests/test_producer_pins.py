"""Pins of the producer oracle (oracle/producer.py) against what the definition
fixes: an independent loop formulation, closed forms for zero and bias-only
projections, softmax invariants, and central finite differences for the
backward. CPU only.
"""
import numpy as np
import pytest

from oracle import producer
from scale_deformable_attention_forward_amd.workloads import make_producer_inputs

LEVELS = ((6, 9), (3, 5), (2, 2))


def _inp(seed=0, B=2, N_q=5, N_h=3, N_p=2, D=7, **kw):
    return make_producer_inputs(B, LEVELS, N_q, N_h, N_p, D, seed, **kw)


def _fwd(d, layout="BQHLP2", **over):
    args = dict(query=d["query"], reference_points=d["reference_points"], offset_weight=d["offset_weight"],
                offset_bias=d["offset_bias"], attention_weight=d["attention_weight"],
                attention_bias=d["attention_bias"], spatial_shapes=d["spatial_shapes"], N_h=d["N_h"],
                N_p=d["N_p"], sampling_locations_layout=layout)
    args.update(over)
    return producer.forward(**args)


def test_matches_loop_formulation():
    d = _inp(seed=1)
    loc, attn = _fwd(d)
    loc2, attn2 = producer.forward_loops(d["query"], d["reference_points"], d["offset_weight"], d["offset_bias"],
                                         d["attention_weight"], d["attention_bias"], d["spatial_shapes"],
                                         d["N_h"], d["N_p"])
    np.testing.assert_allclose(loc, loc2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(attn, attn2, rtol=0, atol=1e-14)


def test_zero_projection_gives_reference_points_and_uniform_weights():
    d = _inp(seed=2)
    zero = {k: np.zeros_like(d[k]) for k in ("offset_weight", "offset_bias", "attention_weight", "attention_bias")}
    loc, attn = _fwd(d, **zero)
    B, N_q, N_l = d["reference_points"].shape[:3]
    want = np.broadcast_to(d["reference_points"].astype(np.float64)[:, :, None, :, None, :], loc.shape)
    np.testing.assert_array_equal(loc, want)
    np.testing.assert_array_equal(attn, np.full(attn.shape, 1.0 / (N_l * d["N_p"])))


def test_bias_only_offsets_move_by_whole_pixels():
    """offset = (W_l * dx, H_l * dy) in pixels moves the normalised location by
    exactly (dx, dy): the offsets are divided by the level's (W, H), x by W."""
    d = _inp(seed=3)
    N_h, N_p = d["N_h"], d["N_p"]
    rng = np.random.default_rng(5)
    dxy = rng.uniform(-0.3, 0.3, size=(N_h, len(LEVELS), N_p, 2))
    wh = np.array([[w, h] for h, w in LEVELS], dtype=np.float64)[None, :, None, :]
    bias = (dxy * wh).reshape(-1)
    loc, _ = _fwd(d, offset_weight=np.zeros_like(d["offset_weight"]), offset_bias=bias)
    want = d["reference_points"].astype(np.float64)[:, :, None, :, None, :] + dxy[None, None]
    np.testing.assert_allclose(loc, want, rtol=0, atol=1e-15)


def test_softmax_invariants():
    d = _inp(seed=4)
    _, attn = _fwd(d)
    np.testing.assert_allclose(attn.reshape(*attn.shape[:3], -1).sum(-1), 1.0, rtol=0, atol=1e-15)
    assert (attn > 0).all()
    # a constant added to all logits of a head changes nothing
    N_h, S = d["N_h"], len(LEVELS) * d["N_p"]
    shift = np.repeat(np.arange(N_h, dtype=np.float64) * 3.0 - 2.0, S)
    _, attn2 = _fwd(d, attention_bias=d["attention_bias"] + shift)
    np.testing.assert_allclose(attn2, attn, rtol=1e-13, atol=0)


def test_layouts_are_transposes():
    d = _inp(seed=6)
    a, _ = _fwd(d, "BQHLP2")
    b, _ = _fwd(d, "B2QHLP")
    np.testing.assert_array_equal(np.moveaxis(b, 1, -1), a)


@pytest.mark.parametrize("layout", ["BQHLP2", "B2QHLP"])
def test_backward_matches_finite_differences(layout):
    d = _inp(seed=7, grad_seed=8)
    gl = d["grad_sampling_locations"].astype(np.float64)
    if layout == "B2QHLP":
        gl = np.moveaxis(gl, -1, 1)
    gA = d["grad_attention_weights"].astype(np.float64)
    params = {k: d[k].astype(np.float64) for k in ("query", "reference_points", "offset_weight",
                                                   "offset_bias", "attention_weight", "attention_bias")}

    def loss(p):
        loc, attn = _fwd(d, layout, **p)
        return float((loc * gl).sum() + (attn * gA).sum())

    _, attn = _fwd(d, layout, **params)
    g = producer.backward(params["query"], params["offset_weight"], params["attention_weight"], attn, gl, gA,
                          d["spatial_shapes"], d["N_h"], d["N_p"], layout)
    rng = np.random.default_rng(9)
    eps = 1e-6
    for name, arr in params.items():
        assert g[name].shape == arr.shape, name
        for _ in range(6):
            idx = tuple(rng.integers(s) for s in arr.shape)
            p_hi = {k: v.copy() for k, v in params.items()}
            p_lo = {k: v.copy() for k, v in params.items()}
            p_hi[name][idx] += eps
            p_lo[name][idx] -= eps
            fd = (loss(p_hi) - loss(p_lo)) / (2 * eps)
            assert abs(fd - g[name][idx]) <= 1e-6 * (1 + abs(fd)), (name, idx, fd, g[name][idx])


def test_dyadic_inputs_give_float32_exact_locations():
    """The dyadic draw with power-of-two levels makes every location a float32
    number exactly (the fused kernel's exact-location parity case relies on it)."""
    levels = ((16, 16), (8, 8), (4, 4))
    d = make_producer_inputs(2, levels, 40, 2, 3, 64, 11, dyadic=True)
    loc, attn = producer.forward(d["query"], d["reference_points"], d["offset_weight"], d["offset_bias"],
                                 d["attention_weight"], d["attention_bias"], levels, 2, 3)
    np.testing.assert_array_equal(loc, loc.astype(np.float32).astype(np.float64))
    assert np.abs(loc).max() < 2.0 and np.isfinite(attn).all()
