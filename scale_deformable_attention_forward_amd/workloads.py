"""Seeded synthetic workloads for multi-scale deformable attention.

This module only draws inputs: it holds none of the method's arithmetic, and
both the HIP path's tests/benchmark and the CPU oracle's tests take their
inputs from it.

Recipe (numpy ``default_rng(seed)``, draws in this order):
  1. value ~ N(0, 1), drawn as (B, L, N_h, C_h) and cast to float32; the BNLC
     layout is the transpose of the same numbers; bfloat16 values are the
     round-to-nearest-even bfloat16 of those float32 numbers.
  2. sampling locations, drawn as (B, N_q, N_h, N_l, N_p, 2) in float64 and
     cast to float32; B2QHLP is the transpose of the same numbers.
     Distributions: "uniform" U[lo, hi]; "clustered": a per-(b, q) centre
     U[0, 1]^2 plus i.i.d. N(0, 0.02) offsets per (h, l, p, coordinate), not
     clipped.
  3. attention-weight logits ~ N(0, 1), softmax over the N_l * N_p axis of
     each (b, q, h) in float64, then cast to float32.
  4. grad_output ~ N(0, 1) of shape (B, N_q, N_h * C_h), float32, drawn from
     its own generator when a seed for it is given.

The five named workloads are Deformable-DETR-shaped feature pyramids.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ENCODER_LEVELS = ((100, 167), (50, 84), (25, 42), (13, 21))      # L = 22223
SQUARE_LEVELS = ((128, 128), (64, 64), (32, 32), (16, 16))       # L = 21760
TINY_LEVELS = ((8, 8), (4, 4))                                   # L = 80


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    levels: tuple
    N_q: int | None          # None: one query per value pixel (N_q = L)
    N_h: int
    C_h: int
    N_p: int
    seed: int
    loc_dist: str = "uniform"
    loc_range: tuple = (0.0, 1.0)
    value_dtype: str = "fp32"
    value_layout: str = "BLNC"
    sampling_locations_layout: str = "BQHLP2"
    align_corners: bool = False
    padding_mode: str = "zeros"
    grad_seed: int | None = None
    passes: tuple = field(default=("forward",))

    @property
    def L(self) -> int:
        return int(sum(h * w for h, w in self.levels))

    @property
    def num_queries(self) -> int:
        return self.L if self.N_q is None else self.N_q

    @property
    def N_l(self) -> int:
        return len(self.levels)


WORKLOADS = {
    1: Workload("tiny_fp32_fwd_bwd", B=1, levels=TINY_LEVELS, N_q=16, N_h=2, C_h=8, N_p=2, seed=1,
                loc_dist="uniform", loc_range=(0.0, 1.0), grad_seed=101,
                passes=("forward", "backward")),
    2: Workload("encoder_fp32_fwd", B=2, levels=ENCODER_LEVELS, N_q=None, N_h=8, C_h=32, N_p=4,
                seed=2, loc_dist="uniform", loc_range=(-0.05, 1.05)),
    3: Workload("decoder_fp32_fwd", B=8, levels=ENCODER_LEVELS, N_q=300, N_h=8, C_h=32, N_p=4,
                seed=3, loc_dist="clustered"),
    4: Workload("square_bf16_bnlc_b2qhlp_align_border_fwd", B=4, levels=SQUARE_LEVELS, N_q=None,
                N_h=8, C_h=32, N_p=4, seed=4, loc_dist="uniform", loc_range=(-0.05, 1.05),
                value_dtype="bf16", value_layout="BNLC", sampling_locations_layout="B2QHLP",
                align_corners=True, padding_mode="border"),
    5: Workload("encoder_fp32_bwd", B=2, levels=ENCODER_LEVELS, N_q=None, N_h=8, C_h=32, N_p=4,
                seed=2, loc_dist="uniform", loc_range=(-0.05, 1.05), grad_seed=5,
                passes=("backward",)),
}


# The producer of locations and weights at the encoder shape, with the
# feature width of Deformable-DETR-style encoders (D = N_h * C_h = 256).
PRODUCER_WORKLOAD = dict(B=2, levels=ENCODER_LEVELS, N_q=22223, N_h=8, N_p=4, C_h=32, D=256, seed=61)


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def level_start_index(levels) -> tuple:
    starts, acc = [], 0
    for h, w in levels:
        starts.append(acc)
        acc += h * w
    return tuple(starts)


def make_inputs(B, levels, N_q, N_h, C_h, N_p, seed, loc_dist="uniform", loc_range=(0.0, 1.0),
                value_dtype="fp32", value_layout="BLNC", sampling_locations_layout="BQHLP2",
                grad_seed=None):
    """Draw one problem. Returns a dict of numpy arrays plus the level tables.

    ``value`` is float32 (the exact values of the bfloat16 numbers when
    value_dtype == "bf16"); ``value_bf16_bits`` holds the uint16 patterns then.
    """
    levels = tuple((int(h), int(w)) for h, w in levels)
    L = sum(h * w for h, w in levels)
    N_l = len(levels)
    rng = np.random.default_rng(seed)
    value = rng.standard_normal((B, L, N_h, C_h)).astype(np.float32)
    if loc_dist == "uniform":
        lo, hi = loc_range
        loc = rng.uniform(lo, hi, size=(B, N_q, N_h, N_l, N_p, 2))
    elif loc_dist == "clustered":
        centre = rng.uniform(0.0, 1.0, size=(B, N_q, 1, 1, 1, 2))
        loc = centre + rng.normal(0.0, 0.02, size=(B, N_q, N_h, N_l, N_p, 2))
    else:
        raise ValueError(f"unknown location distribution {loc_dist!r}")
    loc = loc.astype(np.float32)
    logits = rng.standard_normal((B, N_q, N_h, N_l * N_p))
    logits -= logits.max(axis=-1, keepdims=True)
    e = np.exp(logits)
    attn = (e / e.sum(axis=-1, keepdims=True)).astype(np.float32).reshape(B, N_q, N_h, N_l, N_p)
    out = {}
    if value_dtype == "bf16":
        bits = bf16_round_bits(value)
        value = bf16_bits_to_f32(bits)
        if value_layout == "BNLC":
            bits = np.ascontiguousarray(bits.transpose(0, 2, 1, 3))
        out["value_bf16_bits"] = bits
    elif value_dtype != "fp32":
        raise ValueError(f"unknown value dtype {value_dtype!r}")
    if value_layout == "BNLC":
        value = np.ascontiguousarray(value.transpose(0, 2, 1, 3))
    if sampling_locations_layout == "B2QHLP":
        loc = np.ascontiguousarray(loc.transpose(0, 5, 1, 2, 3, 4))
    out.update(value=value, sampling_locations=loc, attention_weights=attn,
               spatial_shapes=levels, level_start_index=level_start_index(levels),
               value_dtype=value_dtype, value_layout=value_layout,
               sampling_locations_layout=sampling_locations_layout)
    if grad_seed is not None:
        g = np.random.default_rng(grad_seed).standard_normal((B, N_q, N_h * C_h)).astype(np.float32)
        if value_dtype == "bf16":
            g = bf16_bits_to_f32(bf16_round_bits(g))
        out["grad_output"] = g
    return out


def make_large_value(B, L, N_h, C_h, seed, value_dtype="fp32", chunk=1 << 25):
    """value ~ N(0, 1) of shape (B, L, N_h, C_h) for tensors of gigabytes:
    drawn from ``default_rng(seed)`` directly in float32, ``chunk`` elements
    at a time (the named workloads draw float64 first; that would need eight
    bytes per element of host memory here). Returns (value float32,
    bfloat16 bit patterns or None); with value_dtype "bf16" the float32
    array holds the exact values of the round-to-nearest-even bfloat16
    numbers."""
    rng = np.random.default_rng(seed)
    n = B * L * N_h * C_h
    value = np.empty(n, dtype=np.float32)
    bits = np.empty(n, dtype=np.uint16) if value_dtype == "bf16" else None
    for i in range(0, n, chunk):
        part = rng.standard_normal(min(chunk, n - i), dtype=np.float32)
        if bits is not None:
            b = bf16_round_bits(part)
            bits[i:i + len(part)] = b
            part = bf16_bits_to_f32(b)
        value[i:i + len(part)] = part
    shape = (B, L, N_h, C_h)
    return value.reshape(shape), (None if bits is None else bits.reshape(shape))


def make_workload(wl: Workload | int, grad_seed=None):
    """Inputs for a named workload (or its number), plus its mode flags."""
    if isinstance(wl, int):
        wl = WORKLOADS[wl]
    g = wl.grad_seed if grad_seed is None else grad_seed
    d = make_inputs(wl.B, wl.levels, wl.num_queries, wl.N_h, wl.C_h, wl.N_p, wl.seed,
                    loc_dist=wl.loc_dist, loc_range=wl.loc_range, value_dtype=wl.value_dtype,
                    value_layout=wl.value_layout,
                    sampling_locations_layout=wl.sampling_locations_layout, grad_seed=g)
    d.update(align_corners=wl.align_corners, padding_mode=wl.padding_mode)
    return d


def make_producer_inputs(B, levels, N_q, N_h, N_p, D, seed, value_dtype="fp32", offset_pixels=2.0,
                         grad_seed=None, dyadic=False):
    """Draw the inputs of the producer of sampling locations and attention
    weights: query features ~ N(0, 1) of shape (B, N_q, D), reference points
    U[0, 1] of shape (B, N_q, N_l, 2), an offset projection (N_h*N_l*N_p*2, D)
    whose outputs are about `offset_pixels` pixels, an attention projection
    (N_h*N_l*N_p, D) with logits of about unit size, and small biases. With
    value_dtype "bf16" the query and both projections are rounded to bfloat16
    (``*_bf16_bits`` hold the patterns; the float32 arrays hold their exact
    values). With grad_seed, also N(0, 1) gradients for the two outputs.

    dyadic=True draws coarse dyadic numbers instead (query integers in
    [-2, 2], offset weights k/64 and attention weights k/256 with integer
    |k| <= 4, biases k/64, reference points k/256): for D <= 64 every product
    and partial sum of the projection then fits a float32 mantissa, and with
    power-of-two level sizes so does reference + offset / size.
    """
    levels = tuple((int(h), int(w)) for h, w in levels)
    N_l = len(levels)
    S = N_l * N_p
    rng = np.random.default_rng(seed)
    if dyadic:
        out = {
            "query": rng.integers(-2, 3, size=(B, N_q, D)).astype(np.float32),
            "reference_points": (rng.integers(0, 257, size=(B, N_q, N_l, 2)) / 256.0).astype(np.float32),
            "offset_weight": (rng.integers(-4, 5, size=(N_h * S * 2, D)) / 64.0).astype(np.float32),
            "offset_bias": (rng.integers(-64, 65, size=N_h * S * 2) / 64.0).astype(np.float32),
            "attention_weight": (rng.integers(-4, 5, size=(N_h * S, D)) / 256.0).astype(np.float32),
            "attention_bias": (rng.integers(-16, 17, size=N_h * S) / 64.0).astype(np.float32),
        }
    else:
        out = {
            "query": rng.standard_normal((B, N_q, D)).astype(np.float32),
            "reference_points": rng.uniform(0.0, 1.0, size=(B, N_q, N_l, 2)).astype(np.float32),
            "offset_weight": (rng.standard_normal((N_h * S * 2, D)) * (offset_pixels / np.sqrt(D))).astype(np.float32),
            "offset_bias": rng.normal(0.0, offset_pixels, size=N_h * S * 2).astype(np.float32),
            "attention_weight": (rng.standard_normal((N_h * S, D)) / np.sqrt(D)).astype(np.float32),
            "attention_bias": rng.normal(0.0, 0.1, size=N_h * S).astype(np.float32),
        }
    if value_dtype == "bf16":
        for k in ("query", "offset_weight", "attention_weight"):
            bits = bf16_round_bits(out[k])
            out[k] = bf16_bits_to_f32(bits)
            out[k + "_bf16_bits"] = bits
    elif value_dtype != "fp32":
        raise ValueError(f"unknown value dtype {value_dtype!r}")
    out.update(spatial_shapes=levels, level_start_index=level_start_index(levels), N_h=N_h, N_p=N_p, D=D,
               value_dtype=value_dtype)
    if grad_seed is not None:
        g = np.random.default_rng(grad_seed)
        out["grad_sampling_locations"] = g.standard_normal((B, N_q, N_h, N_l, N_p, 2)).astype(np.float32)
        out["grad_attention_weights"] = g.standard_normal((B, N_q, N_h, N_l, N_p)).astype(np.float32)
    return out
