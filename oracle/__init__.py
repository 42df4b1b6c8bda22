"""CPU oracle for multi-scale deformable attention.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers allowed. The HIP
library and its Python binding never import this package, and this package
imports nothing from them.

``forward``/``backward`` wrap the plain-C fp64 implementation in
``msda_oracle.c`` (the definition written out, see its header for the passages
of "MS Deformable Attention Kernel API Reference" and "MS Deformable Attention
Backward Kernel API Reference" it follows). ``bruteforce`` holds a second,
independent dense tent-sum formulation for tiny inputs.

Every array argument is converted to float64 (an exact upcast for float32 and
bfloat16 inputs). Layout and mode arguments take the pages' strings.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

VALUE_LAYOUTS = {"BLNC": 0, "BNLC": 1}
LOC_LAYOUTS = {"BQHLP2": 0, "B2QHLP": 1}
PADDINGS = {"zeros": 0, "border": 1}

_lib = None


def build_oracle() -> str:
    """Compile msda_oracle.c into liboracle.so with gcc (IEEE, no fast-math)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build_oracle()
    _lib = bind(_LIB)
    return _lib


def bind(path):
    """Load an oracle build from ``path`` and declare its C signatures."""
    lib = ctypes.CDLL(path)
    i64, i32 = ctypes.c_int64, ctypes.c_int
    p64 = ctypes.POINTER(ctypes.c_int64)
    pd = ctypes.c_void_p
    common = [i64] * 7 + [p64, p64] + [i32] * 5
    lib.oracle_forward.argtypes = common + [pd, pd, pd, pd]
    lib.oracle_forward.restype = i32
    lib.oracle_backward.argtypes = common + [pd] * 7
    lib.oracle_backward.restype = i32
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_set_threads.restype = None
    return lib


def max_threads() -> int:
    """Threads the oracle's OpenMP loops use on this host."""
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> None:
    """Threads for later oracle calls (for timing; the results do not depend on it:
    every output element is summed by one thread in a fixed order)."""
    _load().oracle_set_threads(int(n))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _levels(spatial_shapes, level_start_index):
    ss = np.ascontiguousarray(np.asarray(spatial_shapes, dtype=np.int64).reshape(-1, 2))
    ls = np.ascontiguousarray(np.asarray(level_start_index, dtype=np.int64).reshape(-1))
    return ss, ls


def _dims(value, loc, value_layout, loc_layout):
    if value_layout == "BLNC":
        B, L, Nh, Ch = value.shape
    else:
        B, Nh, L, Ch = value.shape
    if loc_layout == "BQHLP2":
        _, Nq, _, Nl, Np, _ = loc.shape
    else:
        _, _, Nq, _, Nl, Np = loc.shape
    return B, L, Nq, Nh, Ch, Nl, Np


def _call_args(dims, ss, ls, value_layout, loc_layout, align_corners, padding_mode, coord_fp32):
    i64p = ctypes.POINTER(ctypes.c_int64)
    return list(dims) + [ss.ctypes.data_as(i64p), ls.ctypes.data_as(i64p),
                         VALUE_LAYOUTS[value_layout], LOC_LAYOUTS[loc_layout],
                         int(bool(align_corners)), PADDINGS[padding_mode], int(bool(coord_fp32))]


def forward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
            value_layout="BLNC", sampling_locations_layout="BQHLP2", align_corners=False,
            padding_mode="zeros", coord_fp32=True):
    """fp64 forward. Returns out of shape (B, N_q, N_h * C_h), float64."""
    lib = _load()
    v, loc, a = _f64(value), _f64(sampling_locations), _f64(attention_weights)
    ss, ls = _levels(spatial_shapes, level_start_index)
    dims = _dims(v, loc, value_layout, sampling_locations_layout)
    B, L, Nq, Nh, Ch, Nl, Np = dims
    out = np.zeros((B, Nq, Nh * Ch), dtype=np.float64)
    rc = lib.oracle_forward(*_call_args(dims, ss, ls, value_layout, sampling_locations_layout,
                                        align_corners, padding_mode, coord_fp32),
                            _ptr(v), _ptr(loc), _ptr(a), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_forward rejected the problem (code {rc})")
    return out


def backward(grad_output, value, spatial_shapes, level_start_index, sampling_locations,
             attention_weights, value_layout="BLNC", sampling_locations_layout="BQHLP2",
             align_corners=False, padding_mode="zeros", compute_grad_value=True,
             compute_grad_sampling_locations=True, compute_grad_attention_weights=True,
             coord_fp32=True):
    """fp64 backward. Returns (grad_value, grad_sampling_locations,
    grad_attention_weights), each float64 in its input's layout, None where
    the matching compute flag is False."""
    lib = _load()
    g, v = _f64(grad_output), _f64(value)
    loc, a = _f64(sampling_locations), _f64(attention_weights)
    ss, ls = _levels(spatial_shapes, level_start_index)
    dims = _dims(v, loc, value_layout, sampling_locations_layout)
    gv = np.zeros(v.shape, np.float64) if compute_grad_value else None
    gl = np.zeros(loc.shape, np.float64) if compute_grad_sampling_locations else None
    ga = np.zeros(a.shape, np.float64) if compute_grad_attention_weights else None
    rc = lib.oracle_backward(*_call_args(dims, ss, ls, value_layout, sampling_locations_layout,
                                         align_corners, padding_mode, coord_fp32),
                             _ptr(g), _ptr(v), _ptr(loc), _ptr(a), _ptr(gv), _ptr(gl), _ptr(ga))
    if rc != 0:
        raise ValueError(f"oracle_backward rejected the problem (code {rc})")
    return gv, gl, ga
