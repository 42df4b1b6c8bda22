"""Dense tent-sum brute force for multi-scale deformable attention (tiny inputs).

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).

This is a second formulation of the forward and of grad_value that shares no
floor/corner logic with ``msda_oracle.c``. Bilinear interpolation of a level
at pixel coordinate (x, y) is written as the separable tent sum

    S[c] = sum_{i < H, j < W} max(0, 1 - |x - j|) * max(0, 1 - |y - i|) * V[i, j, c]

("MS Deformable Attention Kernel API Reference", Background: bilinear
interpolation of each level; the tent sum equals the four-corner form because
at most two tents per axis are nonzero). Zeros padding is the restriction of
the sum to in-range pixels; border padding first clamps (x, y) into
[0, W-1] x [0, H-1] (the page's Parameters "padding_mode").

For every (b, h, l) a dense matrix M (samples x pixels of the level) is
formed, the forward is M @ V_l and grad_value is M^T @ (A * G): the adjoint of
the forward ("MS Deformable Attention Backward Kernel API Reference",
Returns). grad_attention_weights is <G, M @ V_l>.

Layouts are handled by numpy transposes to BLNC / BQHLP2 and back. The
coordinate map is binary64 throughout (``coord="fp64"``) or, with
``coord="fp32"``, the binary64 value of loc*W - 0.5 (resp. loc*(W-1)) rounded
once to binary32.
"""
from __future__ import annotations

import numpy as np


def _to_blnc(value, layout):
    v = np.asarray(value, dtype=np.float64)
    return v if layout == "BLNC" else v.transpose(0, 2, 1, 3)


def _to_bqhlp2(loc, layout):
    a = np.asarray(loc, dtype=np.float64)
    return a if layout == "BQHLP2" else a.transpose(0, 2, 3, 4, 5, 1)


def _pixel(loc, size, align_corners, padding_mode, coord):
    if align_corners:
        x = loc * (size - 1)
    else:
        x = loc * size - 0.5
    if coord == "fp32":
        x = x.astype(np.float32).astype(np.float64)
    if padding_mode == "border":
        x = np.clip(x, 0.0, size - 1)
    return x


def _tent_matrix(x, y, H, W):
    """(n, H*W) matrix of bilinear weights, row-major pixels (row i, col j)."""
    j = np.arange(W, dtype=np.float64)
    i = np.arange(H, dtype=np.float64)
    wx = np.maximum(0.0, 1.0 - np.abs(x[:, None] - j[None, :]))  # (n, W)
    wy = np.maximum(0.0, 1.0 - np.abs(y[:, None] - i[None, :]))  # (n, H)
    return (wy[:, :, None] * wx[:, None, :]).reshape(len(x), H * W)


def _level_matrices(loc6, spatial_shapes, align_corners, padding_mode, coord):
    """Yield (l, start, H, W, Mfun) where Mfun(b, h) is the (N_q*N_p, H*W) matrix."""
    start = 0
    for l, (H, W) in enumerate(np.asarray(spatial_shapes, dtype=np.int64).reshape(-1, 2)):
        H, W = int(H), int(W)

        def mfun(b, h, l=l, H=H, W=W):
            lx = loc6[b, :, h, l, :, 0].reshape(-1)
            ly = loc6[b, :, h, l, :, 1].reshape(-1)
            x = _pixel(lx, W, align_corners, padding_mode, coord)
            y = _pixel(ly, H, align_corners, padding_mode, coord)
            return _tent_matrix(x, y, H, W)

        yield l, start, H, W, mfun
        start += H * W


def forward(value, spatial_shapes, sampling_locations, attention_weights, value_layout="BLNC",
            sampling_locations_layout="BQHLP2", align_corners=False, padding_mode="zeros",
            coord="fp64"):
    v = _to_blnc(value, value_layout)
    loc = _to_bqhlp2(sampling_locations, sampling_locations_layout)
    A = np.asarray(attention_weights, dtype=np.float64)
    B, L, Nh, Ch = v.shape
    _, Nq, _, Nl, Np, _ = loc.shape
    out = np.zeros((B, Nq, Nh, Ch))
    for l, start, H, W, mfun in _level_matrices(loc, spatial_shapes, align_corners, padding_mode, coord):
        for b in range(B):
            for h in range(Nh):
                M = mfun(b, h)                                   # (Nq*Np, HW)
                S = (M @ v[b, start:start + H * W, h, :]).reshape(Nq, Np, Ch)
                out[b, :, h, :] += np.einsum("qp,qpc->qc", A[b, :, h, l, :], S)
    return out.reshape(B, Nq, Nh * Ch)


def backward_value_attn(grad_output, value, spatial_shapes, sampling_locations, attention_weights,
                        value_layout="BLNC", sampling_locations_layout="BQHLP2",
                        align_corners=False, padding_mode="zeros", coord="fp64"):
    """Returns (grad_value in value_layout, grad_attention_weights)."""
    v = _to_blnc(value, value_layout)
    loc = _to_bqhlp2(sampling_locations, sampling_locations_layout)
    A = np.asarray(attention_weights, dtype=np.float64)
    B, L, Nh, Ch = v.shape
    _, Nq, _, Nl, Np, _ = loc.shape
    G = np.asarray(grad_output, dtype=np.float64).reshape(B, Nq, Nh, Ch)
    gv = np.zeros_like(v)
    ga = np.zeros(A.shape)
    for l, start, H, W, mfun in _level_matrices(loc, spatial_shapes, align_corners, padding_mode, coord):
        for b in range(B):
            for h in range(Nh):
                M = mfun(b, h)
                S = (M @ v[b, start:start + H * W, h, :]).reshape(Nq, Np, Ch)
                ga[b, :, h, l, :] = np.einsum("qc,qpc->qp", G[b, :, h, :], S)
                R = (A[b, :, h, l, :][:, :, None] * G[b, :, h, :][:, None, :]).reshape(Nq * Np, Ch)
                gv[b, start:start + H * W, h, :] += M.T @ R
    if value_layout == "BNLC":
        gv = gv.transpose(0, 2, 1, 3)
    return np.ascontiguousarray(gv), ga
