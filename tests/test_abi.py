"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad problems on the host before any HIP call
(so these calls enqueue nothing and touch no device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msda.h")

torch = pytest.importorskip("torch")
from scale_deformable_attention_forward_amd import binding  # noqa: E402


class _NoLaunchLib:
    """The library with every msda_* call checked: no call in this module may
    get as far as a HIP call. Without a GPU a launch returns MSDA_ERR_HIP (6),
    so a call that passed host validation by mistake fails here on the CPU
    instead of launching a kernel on the fake addresses below on a GPU host."""

    def __init__(self, lib):
        self._lib = lib

    def __getattr__(self, name):
        fn = getattr(self._lib, name)
        if not name.startswith("msda_") or name in ("msda_status_string", "msda_abi_version"):
            return fn

        def checked(*args):
            status = fn(*args)
            assert status != 6, f"{name} reached a HIP call (MSDA_ERR_HIP) in a no-device ABI test"
            return status
        return checked


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from scale_deformable_attention_forward_amd.build import build_library
        build_library()
    return _NoLaunchLib(binding.load_library())


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:msda_status|const char\*|int)\s+(msda_\w+)\s*\(", text, re.M)))


def test_header_declarations_are_exported(lib):
    names = _declared_functions()
    assert set(names) == set(binding.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert lib.msda_abi_version() == binding.ABI_VERSION == 3
    for code, name in binding.STATUS_NAMES.items():
        assert lib.msda_status_string(code).decode().startswith(name)
    assert lib.msda_status_string(99) is not None


LEVELS = ((4, 6), (2, 3))
STARTS = (0, 24)


def _prob(**kw):
    args = dict(B=1, L=30, N_q=5, N_h=2, C_h=8, spatial_shapes=LEVELS, level_start_index=STARTS, N_p=2)
    over = {k: kw.pop(k) for k in list(kw) if k in args}
    args.update(over)
    return binding.make_problem(**args, **kw)


# Fake but well-aligned, non-overlapping device addresses: every call below must
# fail validation before it could dereference them.
P = {k: ctypes.c_void_p(0x10_0000_0000 + i * 0x1_0000_0000) for i, k in
     enumerate(["value", "loc", "attn", "out", "gout", "gv", "gl", "ga"])}


def _fwd(lib, prob, value=P["value"], loc=P["loc"], attn=P["attn"], out=P["out"]):
    return lib.msda_forward(ctypes.byref(prob), value, loc, attn, out, None)


def _bwd(lib, prob, gv=P["gv"], gl=P["gl"], ga=P["ga"], gout=P["gout"], value=P["value"], flags=0,
         ws=None, ws_bytes=0):
    return lib.msda_backward(ctypes.byref(prob), gout, value, P["loc"], P["attn"], gv, gl, ga,
                             flags, ws, ws_bytes, None)


def test_null_problem(lib):
    assert lib.msda_forward(None, P["value"], P["loc"], P["attn"], P["out"], None) == 1
    assert lib.msda_backward(None, P["gout"], P["value"], P["loc"], P["attn"], P["gv"], P["gl"],
                             P["ga"], 0, None, 0, None) == 1
    sz = ctypes.c_size_t(7)
    assert lib.msda_backward_workspace_size(None, ctypes.byref(sz)) == 1


@pytest.mark.parametrize("field,val,code", [
    ("B", -1, 1), ("N_q", -1, 1), ("N_h", 0, 1), ("C_h", 0, 1), ("N_p", 0, 1), ("L", 0, 1),
    ("value_layout", 2, 1), ("sampling_locations_layout", 5, 1), ("align_corners", 2, 1),
    ("padding_mode", 3, 1), ("value_dtype", 9, 1)])
def test_bad_fields(lib, field, val, code):
    prob, keep = _prob()
    setattr(prob, field, val)
    assert _fwd(lib, prob) == code
    assert _bwd(lib, prob) == code


@pytest.mark.parametrize("shapes,starts,L", [
    (((4, 6), (2, 3)), (0, 23), 30),      # start is not the prefix sum
    (((4, 6), (2, 3)), (1, 25), 30),      # first start not 0
    (((4, 6), (2, 3)), (0, 24), 31),      # L != sum H*W
    (((4, 0), (2, 3)), (0, 0), 6),        # W < 1
    (((-1, 6), (2, 3)), (0, -6), 0),      # H < 1 (and L)
])
def test_bad_level_tables(lib, shapes, starts, L):
    prob, keep = _prob(spatial_shapes=shapes, level_start_index=starts, L=L)
    code = _fwd(lib, prob)
    assert code in (1, 2)
    assert code == 2 or L <= 0


def test_too_many_levels(lib):
    shapes = tuple((1, 1) for _ in range(17))
    prob, keep = _prob(spatial_shapes=shapes, level_start_index=tuple(range(17)), L=17)
    assert _fwd(lib, prob) == 4


def test_index_range_limit(lib):
    prob, keep = _prob(B=1 << 20, N_q=1 << 20)
    assert _fwd(lib, prob) == 4


def test_null_and_misaligned_pointers(lib):
    prob, keep = _prob()
    assert _fwd(lib, prob, value=None) == 1
    assert _fwd(lib, prob, out=None) == 1
    assert _fwd(lib, prob, loc=ctypes.c_void_p(P["loc"].value + 2)) == 1
    assert _fwd(lib, prob, out=ctypes.c_void_p(P["out"].value + 1)) == 1


def test_overlapping_output(lib):
    prob, keep = _prob()
    assert _fwd(lib, prob, out=ctypes.c_void_p(P["value"].value + 64)) == 1
    assert _bwd(lib, prob, gl=ctypes.c_void_p(P["value"].value + 128)) == 1
    assert _bwd(lib, prob, ga=ctypes.c_void_p(P["gl"].value + 4)) == 1


def test_nothing_to_compute(lib):
    prob, keep = _prob()
    assert _bwd(lib, prob, gv=None, gl=None, ga=None) == 3


def test_unknown_backward_flags(lib):
    prob, keep = _prob()
    ws = ctypes.c_void_p(0x90_0000_0000)
    assert _bwd(lib, prob, flags=2, ws=ws, ws_bytes=1 << 30) == 1
    assert _bwd(lib, prob, flags=0x80000000, ws=ws, ws_bytes=1 << 30) == 1


def test_workspace_size(lib):
    # C_h = 8: the tiled grad_value pass needs per-sample anchors plus band lists
    prob, keep = _prob()
    sz = ctypes.c_size_t(123)
    assert lib.msda_backward_workspace_size(ctypes.byref(prob), ctypes.byref(sz)) == 0
    samples = 1 * 5 * 2 * 2 * 2
    # a 4 B anchor and a 16 B record per sample, plus band lists of 4 B per
    # entry with at least 2 entries per sample
    assert sz.value >= (20 + 2 * 4) * samples and sz.value % 256 == 0
    # C_h = 6 takes the generic path: no workspace for float32 ...
    prob, keep = _prob(C_h=6)
    assert lib.msda_backward_workspace_size(ctypes.byref(prob), ctypes.byref(sz)) == 0
    assert sz.value == 0
    # ... and a float32 accumulator of value's size for bfloat16
    prob, keep = _prob(C_h=6, value_dtype=torch.bfloat16)
    assert lib.msda_backward_workspace_size(ctypes.byref(prob), ctypes.byref(sz)) == 0
    assert sz.value == 1 * 30 * 2 * 6 * 4
    # bfloat16 with C_h = 8 covers both paths
    prob, keep = _prob(value_dtype=torch.bfloat16)
    assert lib.msda_backward_workspace_size(ctypes.byref(prob), ctypes.byref(sz)) == 0
    assert sz.value >= max((20 + 2 * 4) * samples, 1 * 30 * 2 * 8 * 4)


def test_workspace_size_encoder_shape(lib):
    # 2 x 22223 queries, 8 heads, 4 levels x 4 points, 32 channels: per-sample
    # anchors (4 B), records (16 B), 2 to 4 list entries of 4 B per sample, plus partial
    # tiles of the split coarse levels
    levels = ((100, 167), (50, 84), (25, 42), (13, 21))
    starts = (0, 16700, 20900, 21950)
    prob, keep = binding.make_problem(2, 22223, 22223, 8, 32, levels, starts, 4)
    sz = ctypes.c_size_t(0)
    assert lib.msda_backward_workspace_size(ctypes.byref(prob), ctypes.byref(sz)) == 0
    samples = 2 * 22223 * 8 * 16
    assert (20 + 8) * samples <= sz.value <= (20 + 16) * samples * 1.5


def test_workspace_size_without_samples(lib):
    # no queries: nothing to bucket or tile, and planning the tiles must not
    # divide by the sample count
    for N_q in (0, 1):
        prob, keep = binding.make_problem(1, 30, N_q, 2, 8, ((5, 6),), (0,), 2)
        sz = ctypes.c_size_t(123)
        assert lib.msda_backward_workspace_size(ctypes.byref(prob), ctypes.byref(sz)) == 0


def test_bf16_backward_needs_workspace(lib):
    # the generic path (C_h = 6) accumulates bfloat16 grad_value in float32
    prob, keep = _prob(C_h=6, value_dtype=torch.bfloat16)
    assert _bwd(lib, prob) == 5
    # without grad_value no workspace is needed: validation passes up to the
    # device pointers, so only check the status of a NULL-grad_value call on
    # an empty problem (nothing is launched)
    prob, keep = _prob(C_h=6, value_dtype=torch.bfloat16, N_q=0)
    assert _bwd(lib, prob, gv=None, gout=None, value=None) == 0


def test_workspace_too_small(lib):
    prob, keep = _prob()
    ws = ctypes.c_void_p(0x90_0000_0000)
    assert _bwd(lib, prob, ws=ws, ws_bytes=16) == 5
    assert _bwd(lib, prob) == 5
    # a workspace overlapping an input is rejected
    assert _bwd(lib, prob, ws=P["value"], ws_bytes=1 << 30) == 1


def test_empty_forward_is_noop(lib):
    prob, keep = _prob(N_q=0)
    assert _fwd(lib, prob, value=None, loc=None, attn=None, out=None) == 0
    prob, keep = _prob(B=0)
    assert _fwd(lib, prob, value=None, loc=None, attn=None, out=None) == 0


def test_python_binding_rejects_cpu_tensors(lib):
    v = torch.zeros(1, 30, 2, 8)
    loc = torch.zeros(1, 5, 2, 2, 2, 2)
    a = torch.zeros(1, 5, 2, 2, 2)
    with pytest.raises(ValueError):
        binding.msda_forward(v, LEVELS, STARTS, loc, a)


# ---------------------------------------------------------------- producer ---

Q = {k: ctypes.c_void_p(0x20_0000_0000 + i * 0x1_0000_0000) for i, k in
     enumerate(["query", "ref", "w_off", "b_off", "w_att", "b_att", "loc", "attn", "value", "out",
                "gq", "gref", "gwo", "gbo", "gwa", "gba", "gloc", "gattn", "ws"])}
D_FEAT = 16


def _pfwd(lib, prob, D=D_FEAT, **over):
    a = {k: Q[k] for k in ("query", "ref", "w_off", "b_off", "w_att", "b_att", "loc", "attn")}
    a.update(over)
    return lib.msda_producer_forward(ctypes.byref(prob), D, a["query"], a["ref"], a["w_off"], a["b_off"],
                                     a["w_att"], a["b_att"], a["loc"], a["attn"], None)


def _pfused(lib, prob, D=D_FEAT, **over):
    a = {k: Q[k] for k in ("query", "ref", "w_off", "b_off", "w_att", "b_att", "value", "out", "loc",
                           "attn")}
    a.update(over)
    return lib.msda_fused_forward(ctypes.byref(prob), D, a["query"], a["ref"], a["w_off"], a["b_off"],
                                  a["w_att"], a["b_att"], a["value"], a["out"], a["loc"], a["attn"], None)


def _pbwd(lib, prob, D=D_FEAT, ws_bytes=1 << 30, **over):
    a = {k: Q[k] for k in ("query", "w_off", "w_att", "attn", "gloc", "gattn", "gq", "gref", "gwo", "gbo",
                           "gwa", "gba", "ws")}
    a.update(over)
    return lib.msda_producer_backward(ctypes.byref(prob), D, a["query"], a["w_off"], a["w_att"], a["attn"],
                                      a["gloc"], a["gattn"], a["gq"], a["gref"], a["gwo"], a["gbo"], a["gwa"],
                                      a["gba"], a["ws"], ws_bytes, None)


def test_producer_rejects_bad_arguments(lib):
    prob, keep = _prob()
    assert lib.msda_producer_forward(None, D_FEAT, *[None] * 8, None) == 1
    assert _pfwd(lib, prob, D=0) == 1
    assert _pfwd(lib, prob, query=None) == 1
    assert _pfwd(lib, prob, loc=None) == 1
    assert _pfwd(lib, prob, ref=ctypes.c_void_p(Q["ref"].value + 2)) == 1
    assert _pfwd(lib, prob, attn=ctypes.c_void_p(Q["query"].value + 64)) == 1   # output over an input
    assert _pfused(lib, prob, value=None) == 1
    assert _pfused(lib, prob, out=ctypes.c_void_p(Q["value"].value + 16)) == 1
    assert _pfused(lib, prob, loc=ctypes.c_void_p(Q["out"].value + 16)) == 1


def test_producer_sample_limits(lib):
    # N_l * N_p = 2 * 33 = 66 > 64 for the producer; 2 * 17 = 34 > 32 for the fused kernel
    prob, keep = _prob(N_p=33)
    assert _pfwd(lib, prob) == 4
    prob, keep = _prob(N_p=17)
    assert _pfused(lib, prob) == 4
    # 34 samples are within the producer's limit: validation goes on past the
    # sample check and stops at the missing query pointer (nothing launched)
    assert _pfwd(lib, prob, query=None) == 1


def test_producer_empty_problem_is_noop(lib):
    prob, keep = _prob(N_q=0)
    assert _pfwd(lib, prob, query=None, ref=None, w_off=None, w_att=None, loc=None, attn=None) == 0
    assert _pfused(lib, prob, query=None, value=None, out=None) == 0
    # no rows and no weight gradient asked for: nothing to enqueue
    assert _pbwd(lib, prob, gwo=None, gbo=None, gwa=None, gba=None, query=None, attn=None) == 0


def test_producer_backward_validation(lib):
    prob, keep = _prob()
    assert _pbwd(lib, prob, gq=None, gref=None, gwo=None, gbo=None, gwa=None, gba=None) == 3
    assert _pbwd(lib, prob, ws_bytes=16) == 5
    assert _pbwd(lib, prob, ws=None) == 5
    assert _pbwd(lib, prob, gq=ctypes.c_void_p(Q["query"].value + 4)) == 1
    assert _pbwd(lib, prob, gwa=ctypes.c_void_p(Q["gwo"].value + 4)) == 1
    assert _pbwd(lib, prob, ws=ctypes.c_void_p(Q["ws"].value + 8)) == 1
    assert _pbwd(lib, prob, attn=None) == 1


def test_producer_workspace_size(lib):
    # encoder shape, D = 256: row chunks x heads x 3S projection outputs x (D + 1) floats
    levels = ((100, 167), (50, 84), (25, 42), (13, 21))
    starts = (0, 16700, 20900, 21950)
    prob, keep = binding.make_problem(2, 22223, 22223, 8, 32, levels, starts, 4)
    sz = ctypes.c_size_t(0)
    assert lib.msda_producer_backward_workspace_size(ctypes.byref(prob), 256, ctypes.byref(sz)) == 0
    M = 2 * 22223
    per_chunk = 8 * 48 * 257 * 4
    assert sz.value % per_chunk == 0
    chunks = sz.value // per_chunk
    assert 16 <= chunks <= 64 and chunks * 32 >= M // 64


# ------------------------------------------------------------ no-alloc ---

def _bwd_noalloc(lib, prob, gv=P["gv"], gl=P["gl"], ga=P["ga"], gout=P["gout"], value=P["value"], flags=0):
    return lib.msda_backward_noalloc(ctypes.byref(prob), gout, value, P["loc"], P["attn"], gv, gl, ga, flags, None)


def test_noalloc_validates_like_msda_backward(lib):
    prob, keep = _prob()
    assert _bwd_noalloc(lib, prob, gv=None, gl=None, ga=None) == 3
    assert _bwd_noalloc(lib, prob, flags=2) == 1
    assert _bwd_noalloc(lib, prob, gl=ctypes.c_void_p(P["value"].value + 128)) == 1
    assert _bwd_noalloc(lib, prob, value=None) == 1
    prob.N_h = 0
    assert _bwd_noalloc(lib, prob) == 1


def test_noalloc_rejects_problems_past_its_scratch(lib):
    # 4 x 22223 encoder queries need about twice the 256 MiB static scratch:
    # rejected on the host, nothing enqueued
    levels = ((100, 167), (50, 84), (25, 42), (13, 21))
    starts = (0, 16700, 20900, 21950)
    prob, keep = binding.make_problem(4, 22223, 22223, 8, 32, levels, starts, 4)
    sz = ctypes.c_size_t(0)
    assert lib.msda_backward_workspace_size(ctypes.byref(prob), ctypes.byref(sz)) == 0
    assert sz.value > 256 << 20
    assert _bwd_noalloc(lib, prob) == 5
    # the encoder-sized problem itself fits
    prob, keep = binding.make_problem(2, 22223, 22223, 8, 32, levels, starts, 4)
    assert lib.msda_backward_workspace_size(ctypes.byref(prob), ctypes.byref(sz)) == 0
    assert sz.value <= 256 << 20
