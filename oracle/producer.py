"""CPU oracle of the producer of sampling locations and attention weights.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``): the test
suite, ``__graft_entry__.smoke()`` and the CPU-baseline legs of ``bench.py``
are the only callers; the HIP library never imports it.

"MS Deformable Attention Kernel API Reference" (Background) samples the value
pyramid "at learned sampling locations" with attention weights, and leaves
how they are learned open. The plainest reading, and the one this oracle
writes out in float64, is a linear projection of each query's feature vector
followed by the usual normalisations:

  proj_off[b, q, :]  = query[b, q, :] @ offset_weight.T + offset_bias
                       (offset_weight has shape (N_h * N_l * N_p * 2, D), the
                       output axis ordered (h, l, p, xy))
  proj_att[b, q, :]  = query[b, q, :] @ attention_weight.T + attention_bias
                       (attention_weight has shape (N_h * N_l * N_p, D),
                       ordered (h, l, p))
  sampling_locations[b, q, h, l, p, x] = reference_points[b, q, l, x]
                                         + proj_off[b, q, h, l, p, x] / W_l
  sampling_locations[b, q, h, l, p, y] = reference_points[b, q, l, y]
                                         + proj_off[b, q, h, l, p, y] / H_l
  attention_weights[b, q, h, :, :]     = softmax over the N_l * N_p entries of
                                         proj_att[b, q, h, :, :]

Offsets are in pixels of their level, so dividing by the level's (W, H) turns
them into the normalised coordinates the sampler maps back to pixels. The
weight matrices are (out_features, in_features) like a linear layer.

``backward`` is the exact adjoint of that map (softmax Jacobian, the 1/W, 1/H
scaling, and the two matrix products), in float64.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _normalizer(spatial_shapes, N_h, N_p):
    """(N_h, N_l, N_p, 2) array of (W_l, H_l)."""
    wh = np.array([[w, h] for h, w in spatial_shapes], dtype=np.float64)   # (N_l, 2): (W, H)
    return np.broadcast_to(wh[None, :, None, :], (N_h, len(spatial_shapes), N_p, 2))


def forward(query, reference_points, offset_weight, offset_bias, attention_weight, attention_bias,
            spatial_shapes, N_h, N_p, sampling_locations_layout="BQHLP2"):
    """Returns (sampling_locations, attention_weights) in float64; locations in
    the requested layout, weights (B, N_q, N_h, N_l, N_p)."""
    x = _f64(query)
    B, N_q, D = x.shape
    N_l = len(spatial_shapes)
    S = N_l * N_p
    Wo, Wa = _f64(offset_weight), _f64(attention_weight)
    bo = np.zeros(Wo.shape[0]) if offset_bias is None else _f64(offset_bias)
    ba = np.zeros(Wa.shape[0]) if attention_bias is None else _f64(attention_bias)
    assert Wo.shape == (N_h * S * 2, D) and Wa.shape == (N_h * S, D)
    off = (x.reshape(-1, D) @ Wo.T + bo).reshape(B, N_q, N_h, N_l, N_p, 2)
    logits = (x.reshape(-1, D) @ Wa.T + ba).reshape(B, N_q, N_h, S)
    ref = _f64(reference_points).reshape(B, N_q, 1, N_l, 1, 2)
    loc = ref + off / _normalizer(spatial_shapes, N_h, N_p)
    z = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(z)
    attn = (e / e.sum(axis=-1, keepdims=True)).reshape(B, N_q, N_h, N_l, N_p)
    if sampling_locations_layout == "B2QHLP":
        loc = np.moveaxis(loc, -1, 1)
    return loc, attn


def backward(query, offset_weight, attention_weight, attention_weights, grad_sampling_locations,
             grad_attention_weights, spatial_shapes, N_h, N_p, sampling_locations_layout="BQHLP2"):
    """Gradients of a scalar loss with respect to (query, reference_points,
    offset_weight, offset_bias, attention_weight, attention_bias), given its
    gradients with respect to the producer's two outputs and the forward's
    attention weights. All float64."""
    x = _f64(query)
    B, N_q, D = x.shape
    N_l = len(spatial_shapes)
    S = N_l * N_p
    gl = _f64(grad_sampling_locations)
    if sampling_locations_layout == "B2QHLP":
        gl = np.moveaxis(gl, 1, -1)
    gl = gl.reshape(B, N_q, N_h, N_l, N_p, 2)
    A = _f64(attention_weights).reshape(B, N_q, N_h, S)
    gA = _f64(grad_attention_weights).reshape(B, N_q, N_h, S)
    g_off = (gl / _normalizer(spatial_shapes, N_h, N_p)).reshape(B * N_q, N_h * S * 2)
    g_log = (A * (gA - (A * gA).sum(axis=-1, keepdims=True))).reshape(B * N_q, N_h * S)
    g_ref = gl.sum(axis=(2, 4))                                   # (B, N_q, N_l, 2)
    X = x.reshape(-1, D)
    Wo, Wa = _f64(offset_weight), _f64(attention_weight)
    g_x = (g_off @ Wo + g_log @ Wa).reshape(B, N_q, D)
    return {"query": g_x, "reference_points": g_ref,
            "offset_weight": g_off.T @ X, "offset_bias": g_off.sum(axis=0),
            "attention_weight": g_log.T @ X, "attention_bias": g_log.sum(axis=0)}


def forward_loops(query, reference_points, offset_weight, offset_bias, attention_weight, attention_bias,
                  spatial_shapes, N_h, N_p):
    """The same definition with explicit Python loops and sums (no matrix
    routine, no broadcasting): an independent formulation for tiny inputs."""
    B, N_q, D = len(query), len(query[0]), len(query[0][0])
    N_l = len(spatial_shapes)
    S = N_l * N_p
    loc = np.zeros((B, N_q, N_h, N_l, N_p, 2))
    attn = np.zeros((B, N_q, N_h, N_l, N_p))
    for b in range(B):
        for q in range(N_q):
            xq = [float(v) for v in query[b][q]]
            for h in range(N_h):
                z = []
                for s in range(S):
                    c = h * S + s
                    acc = 0.0 if attention_bias is None else float(attention_bias[c])
                    for d in range(D):
                        acc += xq[d] * float(attention_weight[c][d])
                    z.append(acc)
                mx = max(z)
                ex = [np.exp(v - mx) for v in z]
                tot = sum(ex)
                for s in range(S):
                    l, p = divmod(s, N_p)
                    attn[b, q, h, l, p] = ex[s] / tot
                    H, W = spatial_shapes[l]
                    for xy, norm in ((0, W), (1, H)):
                        c = (h * S + s) * 2 + xy
                        acc = 0.0 if offset_bias is None else float(offset_bias[c])
                        for d in range(D):
                            acc += xq[d] * float(offset_weight[c][d])
                        loc[b, q, h, l, p, xy] = float(reference_points[b][q][l][xy]) + acc / norm
    return loc, attn
