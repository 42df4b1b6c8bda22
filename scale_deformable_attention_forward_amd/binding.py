"""Thin Python binding of the C ABI in include/msda.h (ctypes).

Argument marshalling only: shapes and flags go into an ``msda_problem``,
torch supplies device memory and the current stream, and every step of the
computation runs in the HIP kernels of ``libmsda.so``. There is no fallback:
if the library is missing or a call fails, an exception is raised.

Keyword names and defaults follow "MS Deformable Attention Kernel API
Reference" (API Reference: ms_deformable_attention) and "MS Deformable
Attention Backward Kernel API Reference" (API Reference:
ms_deformable_attention_bwd). The producer calls (sampling locations and
attention weights from query features, alone or fused with the sampler) take
the names of the C declarations in include/msda.h.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsda.so")

MSDA_OK = 0
STATUS_NAMES = {
    0: "MSDA_OK", 1: "MSDA_ERR_INVALID_ARGUMENT", 2: "MSDA_ERR_INVALID_LEVELS",
    3: "MSDA_ERR_NOTHING_TO_COMPUTE", 4: "MSDA_ERR_UNSUPPORTED", 5: "MSDA_ERR_WORKSPACE_TOO_SMALL",
    6: "MSDA_ERR_HIP",
}
VALUE_LAYOUTS = {"BLNC": 0, "BNLC": 1}
LOC_LAYOUTS = {"BQHLP2": 0, "B2QHLP": 1}
PADDINGS = {"zeros": 0, "border": 1}
DTYPES = {torch.float32: 0, torch.bfloat16: 1}
ABI_VERSION = 3
BACKWARD_ACCUMULATE_GRAD_VALUE = 1  # msda_backward flag: grad_value += result

# Every symbol include/msda.h declares.
EXPORTED_SYMBOLS = ("msda_forward", "msda_backward", "msda_backward_workspace_size", "msda_backward_noalloc",
                    "msda_producer_forward", "msda_fused_forward", "msda_producer_backward_workspace_size",
                    "msda_producer_backward", "msda_status_string", "msda_abi_version")


class MsdaProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("L", ctypes.c_int64), ("N_q", ctypes.c_int64),
                ("N_h", ctypes.c_int64), ("C_h", ctypes.c_int64), ("N_l", ctypes.c_int64),
                ("N_p", ctypes.c_int64),
                ("spatial_shapes", ctypes.POINTER(ctypes.c_int64)),
                ("level_start_index", ctypes.POINTER(ctypes.c_int64)),
                ("value_layout", ctypes.c_int32), ("sampling_locations_layout", ctypes.c_int32),
                ("align_corners", ctypes.c_int32), ("padding_mode", ctypes.c_int32),
                ("value_dtype", ctypes.c_int32)]


class MsdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmsda.so and declare its signatures. Raises if it is not built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run `python -m scale_deformable_attention_forward_amd.build` "
                          "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pp = ctypes.POINTER(MsdaProblem)
    lib.msda_forward.argtypes = [pp, vp, vp, vp, vp, vp]
    lib.msda_forward.restype = ctypes.c_int
    lib.msda_backward.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint, vp, sz, vp]
    lib.msda_backward.restype = ctypes.c_int
    lib.msda_backward_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint, vp]
    lib.msda_backward_noalloc.restype = ctypes.c_int
    lib.msda_backward_workspace_size.argtypes = [pp, ctypes.POINTER(sz)]
    lib.msda_backward_workspace_size.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.msda_producer_forward.argtypes = [pp, i64] + [vp] * 8 + [vp]
    lib.msda_producer_forward.restype = ctypes.c_int
    lib.msda_fused_forward.argtypes = [pp, i64] + [vp] * 10 + [vp]
    lib.msda_fused_forward.restype = ctypes.c_int
    lib.msda_producer_backward_workspace_size.argtypes = [pp, i64, ctypes.POINTER(sz)]
    lib.msda_producer_backward_workspace_size.restype = ctypes.c_int
    lib.msda_producer_backward.argtypes = [pp, i64] + [vp] * 12 + [vp, sz, vp]
    lib.msda_producer_backward.restype = ctypes.c_int
    lib.msda_status_string.argtypes = [ctypes.c_int]
    lib.msda_status_string.restype = ctypes.c_char_p
    lib.msda_abi_version.argtypes = []
    lib.msda_abi_version.restype = ctypes.c_int
    if lib.msda_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {lib.msda_abi_version()}, this binding needs "
                          f"{ABI_VERSION}: rebuild the library")
    if path == LIB_PATH:
        _lib = lib
    return lib


def _raise_for(lib, status: int, what: str):
    if status == MSDA_OK:
        return
    msg = f"{what}: {lib.msda_status_string(status).decode()}"
    if status in (1, 2, 3):
        raise ValueError(msg)
    raise MsdaError(status, msg)


def make_problem(B, L, N_q, N_h, C_h, spatial_shapes, level_start_index, N_p,
                 value_layout="BLNC", sampling_locations_layout="BQHLP2", align_corners=False,
                 padding_mode="zeros", value_dtype=torch.float32):
    """Build an MsdaProblem. Returns (problem, keepalive) - keep both alive during the call."""
    ss = [int(v) for hw in spatial_shapes for v in hw]
    ls = [int(v) for v in level_start_index]
    N_l = len(ss) // 2
    if len(ls) != N_l:
        raise ValueError("spatial_shapes and level_start_index differ in length")
    arr_ss = (ctypes.c_int64 * max(1, len(ss)))(*ss)
    arr_ls = (ctypes.c_int64 * max(1, len(ls)))(*ls)
    try:
        vl = VALUE_LAYOUTS[value_layout]
        ll = LOC_LAYOUTS[sampling_locations_layout]
        pm = PADDINGS[padding_mode]
    except KeyError as e:
        raise ValueError(f"unknown layout or padding mode {e}") from None
    if value_dtype not in DTYPES:
        raise ValueError(f"value dtype {value_dtype} not supported (float32 or bfloat16)")
    prob = MsdaProblem(int(B), int(L), int(N_q), int(N_h), int(C_h), N_l, int(N_p), arr_ss, arr_ls,
                       vl, ll, int(bool(align_corners)), pm, DTYPES[value_dtype])
    return prob, (arr_ss, arr_ls)


def _dims(value, sampling_locations, value_layout, sampling_locations_layout):
    if value.dim() != 4:
        raise ValueError("value must be 4-D")
    if value_layout == "BLNC":
        B, L, N_h, C_h = value.shape
    elif value_layout == "BNLC":
        B, N_h, L, C_h = value.shape
    else:
        raise ValueError(f"unknown value_layout {value_layout!r}")
    if sampling_locations.dim() != 6:
        raise ValueError("sampling_locations must be 6-D")
    if sampling_locations_layout == "BQHLP2":
        Bl, N_q, Nh2, N_l, N_p, two = sampling_locations.shape
    elif sampling_locations_layout == "B2QHLP":
        Bl, two, N_q, Nh2, N_l, N_p = sampling_locations.shape
    else:
        raise ValueError(f"unknown sampling_locations_layout {sampling_locations_layout!r}")
    if Bl != B or Nh2 != N_h or two != 2:
        raise ValueError("sampling_locations shape does not match value")
    return B, L, N_q, N_h, C_h, N_l, N_p


def _check_tensor(t, name, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (the library runs on gfx950 only)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_ptr(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def msda_forward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
                 value_layout="BLNC", sampling_locations_layout="BQHLP2", align_corners=False,
                 padding_mode="zeros", output=None, stream=None):
    """Forward sampler: returns (B, N_q, N_h * C_h) in value's dtype."""
    lib = load_library()
    B, L, N_q, N_h, C_h, N_l, N_p = _dims(value, sampling_locations, value_layout,
                                          sampling_locations_layout)
    _check_tensor(value, "value", value.dtype)
    _check_tensor(sampling_locations, "sampling_locations", torch.float32)
    _check_tensor(attention_weights, "attention_weights", torch.float32)
    if tuple(attention_weights.shape) != (B, N_q, N_h, N_l, N_p):
        raise ValueError("attention_weights must have shape (B, N_q, N_h, N_l, N_p)")
    if output is None:
        output = torch.empty((B, N_q, N_h * C_h), dtype=value.dtype, device=value.device)
    else:
        _check_tensor(output, "output", value.dtype)
        if tuple(output.shape) != (B, N_q, N_h * C_h):
            raise ValueError("output must have shape (B, N_q, N_h * C_h)")
    prob, keep = make_problem(B, L, N_q, N_h, C_h, spatial_shapes, level_start_index, N_p,
                              value_layout, sampling_locations_layout, align_corners, padding_mode,
                              value.dtype)
    st = lib.msda_forward(ctypes.byref(prob), value.data_ptr(), sampling_locations.data_ptr(),
                          attention_weights.data_ptr(), output.data_ptr(), _stream_ptr(stream))
    _raise_for(lib, st, "msda_forward")
    return output


def msda_backward(grad_output, value, spatial_shapes, level_start_index, sampling_locations,
                  attention_weights, value_layout="BLNC", sampling_locations_layout="BQHLP2",
                  align_corners=False, padding_mode="zeros", compute_grad_value=True,
                  compute_grad_sampling_locations=True, compute_grad_attention_weights=True,
                  grad_value=None, grad_sampling_locations=None, grad_attention_weights=None,
                  accumulate_grad_value=False, workspace=None, stream=None):
    """Backward: returns (grad_value, grad_sampling_locations, grad_attention_weights), each in
    its input's layout, with None in the slots whose compute flag is False. With
    ``accumulate_grad_value`` the given ``grad_value`` tensor is added to instead of
    overwritten. ``workspace``: a GPU tensor of at least msda_backward_workspace_size
    bytes, None (allocated here), or "static" (msda_backward_noalloc)."""
    lib = load_library()
    B, L, N_q, N_h, C_h, N_l, N_p = _dims(value, sampling_locations, value_layout,
                                          sampling_locations_layout)
    _check_tensor(value, "value", value.dtype)
    _check_tensor(grad_output, "grad_output", value.dtype)
    _check_tensor(sampling_locations, "sampling_locations", torch.float32)
    _check_tensor(attention_weights, "attention_weights", torch.float32)
    if tuple(grad_output.shape) != (B, N_q, N_h * C_h):
        raise ValueError("grad_output must have shape (B, N_q, N_h * C_h)")
    if tuple(attention_weights.shape) != (B, N_q, N_h, N_l, N_p):
        raise ValueError("attention_weights must have shape (B, N_q, N_h, N_l, N_p)")

    def out(flag, given, like, dtype, name):
        if not flag:
            return None
        if given is None:
            return torch.empty(like.shape, dtype=dtype, device=like.device)
        _check_tensor(given, name, dtype)
        if given.shape != like.shape:
            raise ValueError(f"{name} must have the shape of its input")
        return given

    if accumulate_grad_value and compute_grad_value and grad_value is None:
        raise ValueError("accumulate_grad_value needs a grad_value tensor to add to")
    gv = out(compute_grad_value, grad_value, value, value.dtype, "grad_value")
    gl = out(compute_grad_sampling_locations, grad_sampling_locations, sampling_locations,
             torch.float32, "grad_sampling_locations")
    ga = out(compute_grad_attention_weights, grad_attention_weights, attention_weights,
             torch.float32, "grad_attention_weights")
    prob, keep = make_problem(B, L, N_q, N_h, C_h, spatial_shapes, level_start_index, N_p,
                              value_layout, sampling_locations_layout, align_corners, padding_mode,
                              value.dtype)
    ptr = (lambda t: None if t is None else t.data_ptr())
    flags = BACKWARD_ACCUMULATE_GRAD_VALUE if accumulate_grad_value else 0
    if workspace == "static":
        st = lib.msda_backward_noalloc(ctypes.byref(prob), grad_output.data_ptr(), value.data_ptr(),
                                       sampling_locations.data_ptr(), attention_weights.data_ptr(), ptr(gv),
                                       ptr(gl), ptr(ga), flags, _stream_ptr(stream))
        _raise_for(lib, st, "msda_backward_noalloc")
        return gv, gl, ga
    ws_bytes = ctypes.c_size_t(0)
    st = lib.msda_backward_workspace_size(ctypes.byref(prob), ctypes.byref(ws_bytes))
    _raise_for(lib, st, "msda_backward_workspace_size")
    ws = None
    if ws_bytes.value and gv is not None:
        if workspace is not None:
            if workspace.device != value.device or workspace.numel() * workspace.element_size() < ws_bytes.value:
                raise ValueError(f"workspace must be a GPU tensor of at least {ws_bytes.value} bytes")
            ws = workspace
        else:
            ws = torch.empty(ws_bytes.value, dtype=torch.uint8, device=value.device)
    ws_len = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib.msda_backward(ctypes.byref(prob), grad_output.data_ptr(), value.data_ptr(),
                           sampling_locations.data_ptr(), attention_weights.data_ptr(), ptr(gv),
                           ptr(gl), ptr(ga), flags, ptr(ws), ws_len, _stream_ptr(stream))
    _raise_for(lib, st, "msda_backward")
    return gv, gl, ga


def msda_backward_noalloc(grad_output, value, spatial_shapes, level_start_index, sampling_locations,
                          attention_weights, value_layout="BLNC", sampling_locations_layout="BQHLP2",
                          align_corners=False, padding_mode="zeros", compute_grad_value=True,
                          compute_grad_sampling_locations=True, compute_grad_attention_weights=True,
                          grad_value=None, grad_sampling_locations=None, grad_attention_weights=None,
                          accumulate_grad_value=False, stream=None):
    """msda_backward with its workspace in the library's static device scratch
    (for callers that cannot allocate: pass every output tensor). Raises if the
    problem needs more than that scratch holds."""
    return msda_backward(grad_output, value, spatial_shapes, level_start_index, sampling_locations,
                         attention_weights, value_layout, sampling_locations_layout, align_corners,
                         padding_mode, compute_grad_value, compute_grad_sampling_locations,
                         compute_grad_attention_weights, grad_value, grad_sampling_locations,
                         grad_attention_weights, accumulate_grad_value, workspace="static", stream=stream)


class MSDeformableAttention(torch.autograd.Function):
    """torch.autograd wrapper: forward and backward both run in libmsda.so."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
                value_layout="BLNC", sampling_locations_layout="BQHLP2", align_corners=False,
                padding_mode="zeros"):
        ctx.cfg = (tuple(map(tuple, spatial_shapes)), tuple(level_start_index), value_layout,
                   sampling_locations_layout, align_corners, padding_mode)
        ctx.save_for_backward(value, sampling_locations, attention_weights)
        return msda_forward(value, spatial_shapes, level_start_index, sampling_locations,
                            attention_weights, value_layout, sampling_locations_layout,
                            align_corners, padding_mode)

    @staticmethod
    def backward(ctx, grad_out):
        value, loc, attn = ctx.saved_tensors
        ss, ls, vl, ll, ac, pm = ctx.cfg
        need_v, _, _, need_l, need_a = ctx.needs_input_grad[:5]
        if not (need_v or need_l or need_a):
            return (None,) * 9
        gv, gl, ga = msda_backward(grad_out.contiguous(), value, ss, ls, loc, attn, vl, ll, ac, pm,
                                   compute_grad_value=need_v, compute_grad_sampling_locations=need_l,
                                   compute_grad_attention_weights=need_a)
        return gv, None, None, gl, ga, None, None, None, None


def ms_deformable_attention(value, spatial_shapes, level_start_index, sampling_locations,
                            attention_weights, value_layout="BLNC",
                            sampling_locations_layout="BQHLP2", align_corners=False,
                            padding_mode="zeros"):
    """Differentiable multi-scale deformable attention (forward + backward on the GPU)."""
    return MSDeformableAttention.apply(value, spatial_shapes, level_start_index, sampling_locations,
                                       attention_weights, value_layout, sampling_locations_layout,
                                       align_corners, padding_mode)


def backward_workspace_bytes(value, spatial_shapes, level_start_index, sampling_locations,
                             value_layout="BLNC", sampling_locations_layout="BQHLP2",
                             align_corners=False, padding_mode="zeros"):
    """Bytes of workspace msda_backward needs for these shapes (0 if none)."""
    lib = load_library()
    B, L, N_q, N_h, C_h, N_l, N_p = _dims(value, sampling_locations, value_layout,
                                          sampling_locations_layout)
    prob, keep = make_problem(B, L, N_q, N_h, C_h, spatial_shapes, level_start_index, N_p,
                              value_layout, sampling_locations_layout, align_corners, padding_mode,
                              value.dtype)
    n = ctypes.c_size_t(0)
    _raise_for(lib, lib.msda_backward_workspace_size(ctypes.byref(prob), ctypes.byref(n)),
               "msda_backward_workspace_size")
    return n.value


# ------------------------------------------------------------------ producer ---

def _producer_shapes(query, reference_points, offset_weight, attention_weight, spatial_shapes, N_h):
    """(B, N_q, D, N_l, N_p) of a producer call, with its shape checks."""
    if query.dim() != 3:
        raise ValueError("query must have shape (B, N_q, D)")
    B, N_q, D = query.shape
    N_l = len(spatial_shapes)
    rows = attention_weight.shape[0] if attention_weight.dim() == 2 else -1
    if rows <= 0 or rows % (N_h * N_l):
        raise ValueError("attention_weight must have shape (N_h * N_l * N_p, D)")
    N_p = rows // (N_h * N_l)
    if tuple(attention_weight.shape) != (N_h * N_l * N_p, D):
        raise ValueError("attention_weight must have shape (N_h * N_l * N_p, D)")
    if tuple(offset_weight.shape) != (N_h * N_l * N_p * 2, D):
        raise ValueError("offset_weight must have shape (N_h * N_l * N_p * 2, D)")
    if tuple(reference_points.shape) != (B, N_q, N_l, 2):
        raise ValueError("reference_points must have shape (B, N_q, N_l, 2)")
    return B, N_q, D, N_l, N_p


def _check_optional(t, name, shape, dtype):
    if t is None:
        return
    _check_tensor(t, name, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}")


def _producer_inputs(query, reference_points, offset_weight, offset_bias, attention_weight, attention_bias,
                     N_h, N_l, N_p):
    _check_tensor(query, "query", query.dtype)
    if query.dtype not in DTYPES:
        raise ValueError(f"query dtype {query.dtype} not supported (float32 or bfloat16)")
    _check_tensor(reference_points, "reference_points", torch.float32)
    _check_tensor(offset_weight, "offset_weight", query.dtype)
    _check_tensor(attention_weight, "attention_weight", query.dtype)
    _check_optional(offset_bias, "offset_bias", (N_h * N_l * N_p * 2,), torch.float32)
    _check_optional(attention_bias, "attention_bias", (N_h * N_l * N_p,), torch.float32)


def _sampling_shape(B, N_q, N_h, N_l, N_p, layout):
    if layout == "BQHLP2":
        return (B, N_q, N_h, N_l, N_p, 2)
    if layout == "B2QHLP":
        return (B, 2, N_q, N_h, N_l, N_p)
    raise ValueError(f"unknown sampling_locations_layout {layout!r}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def msda_producer_forward(query, reference_points, offset_weight, offset_bias, attention_weight,
                          attention_bias, spatial_shapes, level_start_index, num_heads,
                          sampling_locations_layout="BQHLP2", sampling_locations=None,
                          attention_weights=None, stream=None):
    """Sampling locations (in the requested layout) and attention weights
    (B, N_q, N_h, N_l, N_p) from query features: returns (locations, weights)."""
    lib = load_library()
    N_h = int(num_heads)
    B, N_q, D, N_l, N_p = _producer_shapes(query, reference_points, offset_weight, attention_weight,
                                           spatial_shapes, N_h)
    _producer_inputs(query, reference_points, offset_weight, offset_bias, attention_weight, attention_bias,
                     N_h, N_l, N_p)
    loc_shape = _sampling_shape(B, N_q, N_h, N_l, N_p, sampling_locations_layout)
    if sampling_locations is None:
        sampling_locations = torch.empty(loc_shape, dtype=torch.float32, device=query.device)
    _check_optional(sampling_locations, "sampling_locations", loc_shape, torch.float32)
    if attention_weights is None:
        attention_weights = torch.empty((B, N_q, N_h, N_l, N_p), dtype=torch.float32, device=query.device)
    _check_optional(attention_weights, "attention_weights", (B, N_q, N_h, N_l, N_p), torch.float32)
    L = sum(int(h) * int(w) for h, w in spatial_shapes)
    prob, keep = make_problem(B, L, N_q, N_h, 1, spatial_shapes, level_start_index, N_p, "BLNC",
                              sampling_locations_layout, False, "zeros", query.dtype)
    st = lib.msda_producer_forward(ctypes.byref(prob), D, query.data_ptr(), reference_points.data_ptr(),
                                   offset_weight.data_ptr(), _ptr(offset_bias), attention_weight.data_ptr(),
                                   _ptr(attention_bias), sampling_locations.data_ptr(),
                                   attention_weights.data_ptr(), _stream_ptr(stream))
    _raise_for(lib, st, "msda_producer_forward")
    return sampling_locations, attention_weights


def msda_fused_forward(value, spatial_shapes, level_start_index, query, reference_points, offset_weight,
                       offset_bias, attention_weight, attention_bias, value_layout="BLNC",
                       sampling_locations_layout="BQHLP2", align_corners=False, padding_mode="zeros",
                       return_sampling=False, output=None, stream=None):
    """Producer and sampler in one kernel: returns the (B, N_q, N_h * C_h)
    output, or (output, sampling_locations, attention_weights) with
    ``return_sampling`` (what a backward needs)."""
    lib = load_library()
    if value.dim() != 4:
        raise ValueError("value must be 4-D")
    if value_layout == "BLNC":
        Bv, L, N_h, C_h = value.shape
    elif value_layout == "BNLC":
        Bv, N_h, L, C_h = value.shape
    else:
        raise ValueError(f"unknown value_layout {value_layout!r}")
    B, N_q, D, N_l, N_p = _producer_shapes(query, reference_points, offset_weight, attention_weight,
                                           spatial_shapes, N_h)
    if Bv != B:
        raise ValueError("query and value differ in batch size")
    _check_tensor(value, "value", query.dtype)
    _producer_inputs(query, reference_points, offset_weight, offset_bias, attention_weight, attention_bias,
                     N_h, N_l, N_p)
    if output is None:
        output = torch.empty((B, N_q, N_h * C_h), dtype=value.dtype, device=value.device)
    _check_optional(output, "output", (B, N_q, N_h * C_h), value.dtype)
    loc = attn = None
    if return_sampling:
        loc = torch.empty(_sampling_shape(B, N_q, N_h, N_l, N_p, sampling_locations_layout),
                          dtype=torch.float32, device=value.device)
        attn = torch.empty((B, N_q, N_h, N_l, N_p), dtype=torch.float32, device=value.device)
    prob, keep = make_problem(B, L, N_q, N_h, C_h, spatial_shapes, level_start_index, N_p, value_layout,
                              sampling_locations_layout, align_corners, padding_mode, value.dtype)
    st = lib.msda_fused_forward(ctypes.byref(prob), D, query.data_ptr(), reference_points.data_ptr(),
                                offset_weight.data_ptr(), _ptr(offset_bias), attention_weight.data_ptr(),
                                _ptr(attention_bias), value.data_ptr(), output.data_ptr(), _ptr(loc),
                                _ptr(attn), _stream_ptr(stream))
    _raise_for(lib, st, "msda_fused_forward")
    return (output, loc, attn) if return_sampling else output


PRODUCER_GRADS = ("query", "reference_points", "offset_weight", "offset_bias", "attention_weight",
                  "attention_bias")


def msda_producer_backward(query, offset_weight, attention_weight, attention_weights,
                           grad_sampling_locations, grad_attention_weights, spatial_shapes,
                           level_start_index, sampling_locations_layout="BQHLP2", compute=PRODUCER_GRADS,
                           workspace=None, outputs=None, stream=None):
    """Gradients of the producer's inputs (dict keyed by PRODUCER_GRADS; only
    the names in ``compute`` are computed, the others are None). Either output
    gradient may be None (zero). ``outputs`` may hold preallocated tensors for
    any of the computed gradients."""
    lib = load_library()
    if attention_weights.dim() != 5:
        raise ValueError("attention_weights must have shape (B, N_q, N_h, N_l, N_p)")
    B, N_q, N_h, N_l, N_p = attention_weights.shape
    if N_l != len(spatial_shapes):
        raise ValueError("attention_weights and spatial_shapes differ in level count")
    if query.dim() != 3 or tuple(query.shape[:2]) != (B, N_q):
        raise ValueError("query must have shape (B, N_q, D)")
    D = query.shape[2]
    _check_tensor(query, "query", query.dtype)
    if query.dtype not in DTYPES:
        raise ValueError(f"query dtype {query.dtype} not supported (float32 or bfloat16)")
    _check_optional(offset_weight, "offset_weight", (N_h * N_l * N_p * 2, D), query.dtype)
    _check_optional(attention_weight, "attention_weight", (N_h * N_l * N_p, D), query.dtype)
    _check_tensor(attention_weights, "attention_weights", torch.float32)
    loc_shape = _sampling_shape(B, N_q, N_h, N_l, N_p, sampling_locations_layout)
    _check_optional(grad_sampling_locations, "grad_sampling_locations", loc_shape, torch.float32)
    _check_optional(grad_attention_weights, "grad_attention_weights", (B, N_q, N_h, N_l, N_p), torch.float32)
    unknown = set(compute) - set(PRODUCER_GRADS)
    if unknown:
        raise ValueError(f"unknown gradients {sorted(unknown)}")
    dev = query.device
    shapes = {"query": (query.shape, query.dtype), "reference_points": ((B, N_q, N_l, 2), torch.float32),
              "offset_weight": (offset_weight.shape, torch.float32),
              "offset_bias": ((N_h * N_l * N_p * 2,), torch.float32),
              "attention_weight": (attention_weight.shape, torch.float32),
              "attention_bias": ((N_h * N_l * N_p,), torch.float32)}
    given = outputs or {}
    out = {}
    for k in PRODUCER_GRADS:
        if k not in compute:
            out[k] = None
        elif given.get(k) is not None:
            _check_optional(given[k], f"outputs[{k!r}]", shapes[k][0], shapes[k][1])
            out[k] = given[k]
        else:
            out[k] = torch.empty(shapes[k][0], dtype=shapes[k][1], device=dev)
    L = sum(int(h) * int(w) for h, w in spatial_shapes)
    prob, keep = make_problem(B, L, N_q, N_h, 1, spatial_shapes, level_start_index, N_p, "BLNC",
                              sampling_locations_layout, False, "zeros", query.dtype)
    n = ctypes.c_size_t(0)
    _raise_for(lib, lib.msda_producer_backward_workspace_size(ctypes.byref(prob), D, ctypes.byref(n)),
               "msda_producer_backward_workspace_size")
    ws = None
    if n.value and any(out[k] is not None for k in PRODUCER_GRADS[2:]):
        if workspace is not None:
            if workspace.device != dev or workspace.numel() * workspace.element_size() < n.value:
                raise ValueError(f"workspace must be a GPU tensor of at least {n.value} bytes")
            ws = workspace
        else:
            ws = torch.empty(n.value, dtype=torch.uint8, device=dev)
    ws_len = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib.msda_producer_backward(ctypes.byref(prob), D, query.data_ptr(), offset_weight.data_ptr(),
                                    attention_weight.data_ptr(), attention_weights.data_ptr(),
                                    _ptr(grad_sampling_locations), _ptr(grad_attention_weights),
                                    *(_ptr(out[k]) for k in PRODUCER_GRADS), _ptr(ws), ws_len,
                                    _stream_ptr(stream))
    _raise_for(lib, st, "msda_producer_backward")
    return out


class MSDAProducer(torch.autograd.Function):
    """torch.autograd wrapper of the producer: forward and backward both run in libmsda.so.
    Returns (sampling_locations, attention_weights)."""

    @staticmethod
    def forward(ctx, query, reference_points, offset_weight, offset_bias, attention_weight, attention_bias,
                spatial_shapes, level_start_index, num_heads, sampling_locations_layout="BQHLP2"):
        loc, attn = msda_producer_forward(query, reference_points, offset_weight, offset_bias,
                                          attention_weight, attention_bias, spatial_shapes,
                                          level_start_index, num_heads, sampling_locations_layout)
        ctx.cfg = (tuple(map(tuple, spatial_shapes)), tuple(level_start_index), sampling_locations_layout)
        ctx.save_for_backward(query, offset_weight, attention_weight, attn)
        return loc, attn

    @staticmethod
    def backward(ctx, grad_loc, grad_attn):
        query, w_off, w_att, attn = ctx.saved_tensors
        ss, ls, layout = ctx.cfg
        need = ctx.needs_input_grad[:6]
        names = [k for k, n in zip(PRODUCER_GRADS, need) if n]
        if not names:
            return (None,) * 10
        g = msda_producer_backward(query, w_off, w_att, attn,
                                   None if grad_loc is None else grad_loc.contiguous(),
                                   None if grad_attn is None else grad_attn.contiguous(), ss, ls, layout,
                                   compute=names)
        return tuple(g[k] for k in PRODUCER_GRADS) + (None,) * 4
