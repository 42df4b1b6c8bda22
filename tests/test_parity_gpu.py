"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, element by element, under the comparison rule in
helpers.py. Covers the five named workloads at full size, the flag sweep,
ragged and degenerate shapes, selective gradients and run-to-run stability.
"""
import itertools
import sys

import numpy as np
import pytest

from helpers import RTOL, compare, oracle_backward, oracle_forward, to_device, to_numpy
from scale_deformable_attention_forward_amd.workloads import WORKLOADS, make_inputs, make_workload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _mk(levels=((7, 9), (4, 5), (1, 1)), B=2, N_q=37, N_h=3, C_h=8, N_p=3, seed=0,
        value_dtype="fp32", value_layout="BLNC", loc_layout="BQHLP2", align=False, pad="zeros",
        loc_range=(-0.1, 1.1), grad_seed=1):
    d = make_inputs(B, levels, N_q, N_h, C_h, N_p, seed, loc_range=loc_range, value_dtype=value_dtype,
                    value_layout=value_layout, sampling_locations_layout=loc_layout,
                    grad_seed=grad_seed)
    d.update(align_corners=align, padding_mode=pad)
    return d


def _gpu_forward(d, dev):
    from scale_deformable_attention_forward_amd import msda_forward
    import torch
    t = to_device(d, dev)
    out = msda_forward(t["value"], d["spatial_shapes"], d["level_start_index"], t["sampling_locations"],
                       t["attention_weights"], d["value_layout"], d["sampling_locations_layout"],
                       d["align_corners"], d["padding_mode"])
    torch.cuda.synchronize()
    return to_numpy(out)


def _gpu_backward(d, dev, flags=(True, True, True), **kw):
    from scale_deformable_attention_forward_amd import msda_backward
    import torch
    t = to_device(d, dev)
    res = msda_backward(t["grad_output"], t["value"], d["spatial_shapes"], d["level_start_index"],
                        t["sampling_locations"], t["attention_weights"], d["value_layout"],
                        d["sampling_locations_layout"], d["align_corners"], d["padding_mode"],
                        compute_grad_value=flags[0], compute_grad_sampling_locations=flags[1],
                        compute_grad_attention_weights=flags[2], **kw)
    torch.cuda.synchronize()
    return tuple(to_numpy(r) for r in res)


def _check_forward(d, dev, tag):
    _say(f"forward {tag}")
    got = _gpu_forward(d, dev)
    want = oracle_forward(d)
    return compare(f"forward {tag}", got, want, RTOL[d["value_dtype"]])


def _check_backward(d, dev, tag, flags=(True, True, True)):
    _say(f"backward {tag} flags={flags}")
    got = _gpu_backward(d, dev, flags)
    want = oracle_backward(d, compute_grad_value=flags[0], compute_grad_sampling_locations=flags[1],
                           compute_grad_attention_weights=flags[2])
    names = ("grad_value", "grad_sampling_locations", "grad_attention_weights")
    for n, f, g, w in zip(names, flags, got, want):
        if not f:
            assert g is None
            continue
        compare(f"{n} {tag}", g, w, RTOL[d["value_dtype"]])


# ------------------------------------------------------- named workloads ---

@pytest.mark.parametrize("num", [1, 2, 3, 4])
def test_forward_named_workload_full_size(num, gpu_device):
    wl = WORKLOADS[num]
    d = make_workload(num)
    _check_forward(d, gpu_device, f"workload {num} {wl.name}")


@pytest.mark.parametrize("num", [1, 5])
def test_backward_named_workload_full_size(num, gpu_device):
    wl = WORKLOADS[num]
    d = make_workload(num)
    _check_backward(d, gpu_device, f"workload {num} {wl.name}")


def test_backward_decoder_workload_full_size(gpu_device):
    """The decoder workload's shapes (B=8, N_q=300 clustered queries over the
    L=22223 pyramid) with a grad_output: samples are sparse against the
    pixels, so the tile pass walks the two large levels in pixel mode."""
    d = make_workload(3, grad_seed=1003)
    _check_backward(d, gpu_device, "workload 3 decoder, backward")


# ------------------------------------------------------------- flag sweep ---

SWEEP = list(itertools.product(["BLNC", "BNLC"], ["BQHLP2", "B2QHLP"], [False, True], ["zeros", "border"]))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("mode", SWEEP, ids=lambda m: "-".join(map(str, m)))
def test_forward_flag_sweep(mode, dtype, gpu_device):
    vl, ll, align, pad = mode
    d = _mk(seed=3, value_dtype=dtype, value_layout=vl, loc_layout=ll, align=align, pad=pad)
    _check_forward(d, gpu_device, f"sweep {mode} {dtype}")


@pytest.mark.parametrize("mode", SWEEP, ids=lambda m: "-".join(map(str, m)))
def test_backward_flag_sweep(mode, gpu_device):
    vl, ll, align, pad = mode
    d = _mk(seed=4, value_layout=vl, loc_layout=ll, align=align, pad=pad)
    _check_backward(d, gpu_device, f"sweep {mode}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("mode", SWEEP, ids=lambda m: "-".join(map(str, m)))
def test_backward_flag_sweep_halo_mode(mode, dtype, gpu_device):
    """The sweep on a dense shape (8,000 samples per (b, h, level) against 120
    and 30 pixels: more than one pixel-mode band's worth), so grad_value goes
    through the halo-mode tile kernel, its bands split into chunks, in every
    mode; the default small shapes above take pixel mode."""
    vl, ll, align, pad = mode
    d = _mk(seed=6, levels=((10, 12), (5, 6)), B=1, N_h=2, N_q=2000, C_h=8, N_p=4, value_dtype=dtype,
            value_layout=vl, loc_layout=ll, align=align, pad=pad)
    _check_backward(d, gpu_device, f"sweep halo mode {mode} {dtype}")


# ---------------------------------------------------- shapes and edge cases ---

@pytest.mark.parametrize("C_h", [1, 2, 3, 4, 5, 16, 32, 64, 100, 256, 300])
def test_channel_counts(C_h, gpu_device):
    d = _mk(seed=5, C_h=C_h, N_q=19, N_h=2)
    _check_forward(d, gpu_device, f"C_h={C_h}")
    _check_backward(d, gpu_device, f"C_h={C_h}")


@pytest.mark.parametrize("C_h", [8, 24, 32, 300])
def test_channel_counts_bf16_forward(C_h, gpu_device):
    d = _mk(seed=6, C_h=C_h, N_q=21, N_h=2, value_dtype="bf16", value_layout="BNLC")
    _check_forward(d, gpu_device, f"bf16 C_h={C_h}")


def test_single_level_single_point_single_pixel(gpu_device):
    d = _mk(seed=7, levels=((1, 1),), N_p=1, loc_range=(-1.0, 2.0))
    _check_forward(d, gpu_device, "1x1 level")
    _check_backward(d, gpu_device, "1x1 level")
    d = _mk(seed=7, levels=((1, 1),), N_p=1, pad="border", align=True)
    _check_forward(d, gpu_device, "1x1 level border align")
    _check_backward(d, gpu_device, "1x1 level border align")


def test_sixteen_levels_many_points(gpu_device):
    levels = tuple((1 + (i % 5), 2 + (i * 3) % 7) for i in range(16))
    d = _mk(seed=8, levels=levels, N_p=5, N_q=23)
    _check_forward(d, gpu_device, "16 levels x 5 points (S = 80 > one staging chunk)")
    _check_backward(d, gpu_device, "16 levels x 5 points")


def test_far_out_of_range_locations(gpu_device):
    for pad in ("zeros", "border"):
        d = _mk(seed=9, loc_range=(-50.0, 50.0), pad=pad)
        _check_forward(d, gpu_device, f"far out of range {pad}")
        _check_backward(d, gpu_device, f"far out of range {pad}")


def test_ragged_query_counts(gpu_device):
    for N_q in (1, 2, 31, 33, 65, 257):
        d = _mk(seed=10 + N_q, N_q=N_q, C_h=32, N_h=1, B=1)
        _check_forward(d, gpu_device, f"N_q={N_q}")
        _check_backward(d, gpu_device, f"N_q={N_q}")


@pytest.mark.parametrize("flags", [f for f in itertools.product([True, False], repeat=3) if any(f)])
def test_selective_gradients(flags, gpu_device):
    d = _mk(seed=11)
    _check_backward(d, gpu_device, "selective", flags)


def test_nothing_to_compute_raises(gpu_device):
    d = _mk(seed=12)
    with pytest.raises(ValueError):
        _gpu_backward(d, gpu_device, (False, False, False))


def test_empty_problems(gpu_device):
    import torch
    from scale_deformable_attention_forward_amd import msda_backward, msda_forward
    d = _mk(seed=13, N_q=0)
    t = to_device(d, gpu_device)
    out = msda_forward(t["value"], d["spatial_shapes"], d["level_start_index"], t["sampling_locations"],
                       t["attention_weights"])
    assert out.shape == (2, 0, 24)
    gv_init = torch.full_like(t["value"], 7.0)
    gv, gl, ga = msda_backward(t["grad_output"], t["value"], d["spatial_shapes"], d["level_start_index"],
                               t["sampling_locations"], t["attention_weights"], grad_value=gv_init)
    torch.cuda.synchronize()
    assert gv is gv_init and not gv.any().item()   # nothing sampled: grad_value is all zeros


def test_unaligned_views_take_narrower_vectors(gpu_device):
    """Inputs that start one element into their allocation cannot use 16-byte loads."""
    import torch
    from scale_deformable_attention_forward_amd import msda_forward
    d = _mk(seed=14, C_h=8)
    t = to_device(d, gpu_device)
    v = t["value"]
    buf = torch.empty(v.numel() + 1, dtype=v.dtype, device=gpu_device)
    vv = buf[1:].view(v.shape)
    vv.copy_(v)
    lbuf = torch.empty(t["sampling_locations"].numel() + 1, dtype=torch.float32, device=gpu_device)
    ll = lbuf[1:].view(t["sampling_locations"].shape)
    ll.copy_(t["sampling_locations"])
    out = msda_forward(vv, d["spatial_shapes"], d["level_start_index"], ll, t["attention_weights"])
    torch.cuda.synchronize()
    compare("unaligned", to_numpy(out), oracle_forward(d), RTOL["fp32"])


def test_pixel_centres_are_exact_on_gpu(gpu_device):
    """One-hot weights at pixel centres of power-of-two levels return value bit for bit."""
    levels = ((16, 32), (8, 16), (4, 4))
    d = _mk(seed=15, levels=levels, N_q=40, N_h=2, C_h=32, N_p=2, grad_seed=None)
    B, N_q, N_h, N_l, N_p = d["attention_weights"].shape
    rng = np.random.default_rng(0)
    loc = np.zeros((B, N_q, N_h, N_l, N_p, 2), np.float32)
    A = np.zeros((B, N_q, N_h, N_l, N_p), np.float32)
    want = np.zeros((B, N_q, N_h, 32), np.float32)
    starts = d["level_start_index"]
    for b, q, h in itertools.product(range(B), range(N_q), range(N_h)):
        l, p = rng.integers(N_l), rng.integers(N_p)
        H, W = levels[l]
        i, j = rng.integers(H), rng.integers(W)
        loc[b, q, h] = rng.uniform(0, 1, size=(N_l, N_p, 2))
        loc[b, q, h, l, p] = ((j + 0.5) / W, (i + 0.5) / H)
        A[b, q, h, l, p] = 1.0
        want[b, q, h] = d["value"][b, starts[l] + i * W + j, h]
    d.update(sampling_locations=loc, attention_weights=A)
    got = _gpu_forward(d, gpu_device)
    np.testing.assert_array_equal(got.reshape(want.shape), want)


def test_repeat_runs_are_stable(gpu_device):
    d = _mk(seed=16, C_h=32, N_q=300, N_h=8)
    f1, f2 = _gpu_forward(d, gpu_device), _gpu_forward(d, gpu_device)
    np.testing.assert_array_equal(f1, f2)
    b1, b2 = _gpu_backward(d, gpu_device), _gpu_backward(d, gpu_device)
    for a, b in zip(b1, b2):
        np.testing.assert_array_equal(a, b)   # destination-tiled grad_value: fixed summation order


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_split_bands_are_deterministic(dtype, gpu_device):
    """Coarse levels whose bands are split over many workgroups (partial tiles
    added in chunk order) give bitwise identical grad_value on every run."""
    d = _mk(seed=19, levels=((20, 30), (5, 6), (2, 2)), N_q=6000, N_p=4, B=1, N_h=2, C_h=32,
            value_dtype=dtype)
    runs = [_gpu_backward(d, gpu_device, (True, False, False))[0] for _ in range(3)]
    for r in runs[1:]:
        np.testing.assert_array_equal(runs[0], r)
    compare(f"split bands {dtype}", runs[0], oracle_backward(d, compute_grad_sampling_locations=False,
                                                             compute_grad_attention_weights=False)[0],
            RTOL[dtype])


def test_many_runs_in_one_pass(gpu_device):
    """160,000 samples per (b, h, level) make 79 bucketing runs; on the large
    level every band's list is short, so one pass of the tile pass takes all
    79 runs (more than the 64 a single ballot covers)."""
    d = _mk(levels=((200, 200), (10, 12)), B=1, N_h=1, N_q=40000, C_h=8, N_p=4, seed=29, loc_range=(0.0, 1.0))
    _check_backward(d, gpu_device, "many runs in one pass")


def test_sparse_samples_and_split_band(gpu_device):
    """16,000 samples per (b, h, level) against 18,000 pixels in the large
    level: the tile pass walks that level in pixel mode, and the 6x7 level
    (halo mode) has one band holding every sample of that level, so it is
    split into chunks whose partial tiles the reduction adds."""
    d = _mk(levels=((120, 150), (6, 7)), B=1, N_h=2, N_q=4000, C_h=32, N_p=4, seed=31, loc_range=(-0.05, 1.05))
    _check_backward(d, gpu_device, "sparse shape, split band")


def test_pixel_mode_band_of_many_passes(gpu_device):
    """10,000 samples against the 40,000 pixels of a 200x200 level put it in
    pixel mode, but every location falls in [0, 0.1]^2, so the few bands
    there hold several LDS passes of entries each: every round of pixel
    blocks stages its passes again. Matches the oracle, bitwise the same on
    every run."""
    d = _mk(levels=((200, 200),), B=1, N_h=2, N_q=2500, C_h=8, N_p=4, seed=37, loc_range=(0.0, 0.1))
    _check_backward(d, gpu_device, "pixel mode, many passes per band")
    runs = [_gpu_backward(d, gpu_device, (True, False, False))[0] for _ in range(2)]
    np.testing.assert_array_equal(runs[0], runs[1])


def test_pixel_mode_repeat_runs_are_stable(gpu_device):
    """Decoder-like sparse samples (pixel mode on every level: the two large
    ones have fewer samples than pixels, one band covers the small one):
    grad_value is bitwise the same on every run."""
    d = _mk(levels=((60, 80), (30, 40), (8, 10)), B=2, N_h=4, N_q=200, C_h=32, N_p=4, seed=41,
            loc_range=(-0.05, 1.05))
    runs = [_gpu_backward(d, gpu_device, (True, False, False))[0] for _ in range(3)]
    for r in runs[1:]:
        np.testing.assert_array_equal(runs[0], r)
    compare("pixel mode repeat", runs[0], oracle_backward(d, compute_grad_sampling_locations=False,
                                                          compute_grad_attention_weights=False)[0], RTOL["fp32"])


def _check_pile_up(d, dev, tag, runs=2):
    """Oracle parity of all three gradients, grad_value judged against the
    magnitude of its terms as well (its elements sum thousands of cancelling
    terms), then grad_value bitwise the same on every further run."""
    _say(f"backward {tag}")
    got = _gpu_backward(d, dev)
    want = oracle_backward(d)
    mag = oracle_backward(d, grad_output=np.abs(d["grad_output"]),
                          attention_weights=np.abs(d["attention_weights"]),
                          compute_grad_sampling_locations=False, compute_grad_attention_weights=False)[0]
    rtol = RTOL[d["value_dtype"]]
    compare(f"grad_value {tag}", got[0], want[0], rtol, magnitude=mag)
    compare(f"grad_sampling_locations {tag}", got[1], want[1], rtol)
    compare(f"grad_attention_weights {tag}", got[2], want[2], rtol)
    gv = [_gpu_backward(d, dev, (True, False, False))[0] for _ in range(runs)]
    for r in [got[0]] + gv:
        np.testing.assert_array_equal(gv[0], r)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("pad", ["zeros", "border"])
def test_pile_up_on_one_point(dtype, pad, gpu_device):
    """All 6,000 samples per (b, h) of the 24x30 level at one location: one
    anchor bin holds every entry of its band's three LDS passes (2,048 a
    pass), far past what one lane ranks alone, so whole waves rank them; the
    6x7 level's samples stay spread."""
    d = _mk(levels=((24, 30), (6, 7)), B=1, N_h=2, N_q=1500, C_h=32, N_p=4, seed=43, value_dtype=dtype,
            pad=pad)
    d["sampling_locations"][:, :, :, 0, :, 0] = np.float32(0.4137)
    d["sampling_locations"][:, :, :, 0, :, 1] = np.float32(0.6211)
    _check_pile_up(d, gpu_device, f"pile-up on one point {dtype} {pad}")


def test_pile_up_beside_spread_samples(gpu_device):
    """A quarter of the 32x32 level's samples at one location, the rest
    spread: passes hold one bin of hundreds of entries (ranked by whole
    waves) among bins of a few (ranked by their own lanes), in the same
    waves."""
    d = _mk(levels=((32, 32), (4, 4)), B=1, N_h=2, N_q=2000, C_h=32, N_p=4, seed=61, loc_range=(0.0, 1.0))
    loc = d["sampling_locations"]
    loc[:, ::4, :, 0, :, 0] = np.float32(0.2718)
    loc[:, ::4, :, 0, :, 1] = np.float32(0.5772)
    _check_pile_up(d, gpu_device, "pile-up beside spread samples")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("align", [False, True])
def test_border_clamping_piles_up_on_edges(dtype, align, gpu_device):
    """Border padding with locations in [-1, 2]: two thirds of the samples
    clamp in x, two thirds in y, so each corner pixel of a level takes one
    ninth of them (about 670 per (b, h) on the 24x30 level) and the edge
    pixels tens each. Clamped samples alternate between the two anchors that
    reach their edge pixel with the same weight; the corner bins still pass
    the size one lane ranks alone."""
    d = _mk(levels=((24, 30), (6, 7), (1, 3)), B=1, N_h=2, N_q=1500, C_h=32, N_p=4, seed=47,
            value_dtype=dtype, pad="border", align=align, loc_range=(-1.0, 2.0))
    _check_pile_up(d, gpu_device, f"border pile-up {dtype} align={align}")


def test_border_clamping_in_pixel_mode(gpu_device):
    """The same clamping on a level with fewer samples than pixels (pixel
    mode, one band per level), B2QHLP locations, BNLC value."""
    d = _mk(levels=((60, 80), (12, 16)), B=2, N_h=2, N_q=300, C_h=32, N_p=4, seed=53, pad="border",
            loc_range=(-1.0, 2.0), value_layout="BNLC", loc_layout="B2QHLP")
    _check_pile_up(d, gpu_device, "border pile-up, pixel mode")


def test_autograd_function_matches_oracle(gpu_device):
    import torch
    from scale_deformable_attention_forward_amd import ms_deformable_attention
    d = _mk(seed=17)
    t = to_device(d, gpu_device)
    v = t["value"].clone().requires_grad_(True)
    loc = t["sampling_locations"].clone().requires_grad_(True)
    a = t["attention_weights"].clone().requires_grad_(True)
    out = ms_deformable_attention(v, d["spatial_shapes"], d["level_start_index"], loc, a)
    out.backward(t["grad_output"])
    torch.cuda.synchronize()
    compare("autograd out", to_numpy(out), oracle_forward(d), RTOL["fp32"])
    gv, gl, ga = oracle_backward(d)
    compare("autograd grad_value", to_numpy(v.grad), gv, RTOL["fp32"])
    compare("autograd grad_loc", to_numpy(loc.grad), gl, RTOL["fp32"])
    compare("autograd grad_attn", to_numpy(a.grad), ga, RTOL["fp32"])


@pytest.mark.parametrize("C_h,levels,N_q,N_p,B,N_h", [
    (32, ((16, 20), (8, 10), (4, 5), (2, 3)), 2000, 4, 2, 2),  # several LDS-privatised levels and query chunks
    (64, ((40, 40), (5, 5)), 3200, 4, 1, 1),                   # 64 channels: the big level in channel slices
    (16, ((30, 30), (3, 3)), 1000, 8, 1, 3),
    (8, ((12, 12),), 500, 4, 3, 1),
    (12, ((9, 11), (2, 2)), 700, 3, 1, 2),                     # C_h not a power of two
])
def test_dense_coarse_levels(C_h, levels, N_q, N_p, B, N_h, gpu_device):
    """Many samples per pixel: the coarse levels' grad_value goes through LDS."""
    for vl, pad in (("BLNC", "zeros"), ("BNLC", "border")):
        d = _mk(seed=18, levels=levels, N_q=N_q, N_p=N_p, B=B, N_h=N_h, C_h=C_h, value_layout=vl, pad=pad)
        _check_backward(d, gpu_device, f"dense coarse C_h={C_h} {levels} {vl} {pad}")
        _check_backward(d, gpu_device, f"dense coarse grad_value only C_h={C_h}", (True, False, False))


# ------------------------------------------------------- bfloat16 backward ---

@pytest.mark.parametrize("mode", SWEEP, ids=lambda m: "-".join(map(str, m)))
def test_backward_flag_sweep_bf16(mode, gpu_device):
    vl, ll, align, pad = mode
    d = _mk(seed=20, value_dtype="bf16", value_layout=vl, loc_layout=ll, align=align, pad=pad)
    _check_backward(d, gpu_device, f"bf16 sweep {mode}")


@pytest.mark.parametrize("C_h", [4, 6, 8, 12, 24, 32, 40, 64, 100])
def test_channel_counts_bf16_backward(C_h, gpu_device):
    """C_h % 4 == 0 and <= 64 take the tiled path, the rest the generic one
    (float32 accumulator in the workspace, converted once); on the tiled
    path C_h % 8 == 0 gathers 8 channels a lane (24 and 40 leave lanes of a
    unit idle), the others 4."""
    d = _mk(seed=21, C_h=C_h, N_q=29, N_h=2, value_dtype="bf16")
    _check_backward(d, gpu_device, f"bf16 C_h={C_h}")


def test_backward_bf16_square_workload_full_size(gpu_device):
    """The bfloat16 BNLC / B2QHLP / align_corners / border workload's shapes
    (B=4, 128/64/32/16 square pyramid, N_q = L = 21760) with a grad_output."""
    wl = WORKLOADS[4]
    d = make_inputs(wl.B, wl.levels, wl.L, wl.N_h, wl.C_h, wl.N_p, seed=4, loc_range=wl.loc_range,
                    value_dtype="bf16", value_layout="BNLC", sampling_locations_layout="B2QHLP",
                    grad_seed=24)
    d.update(align_corners=True, padding_mode="border")
    _check_backward(d, gpu_device, "bf16 square pyramid full size")


def test_dense_coarse_levels_bf16(gpu_device):
    d = _mk(seed=22, levels=((16, 20), (8, 10), (4, 5), (2, 3)), N_q=2000, N_p=4, B=2, N_h=2, C_h=32,
            value_dtype="bf16", value_layout="BNLC")
    _check_backward(d, gpu_device, "bf16 dense coarse")


# --------------------------------------------------- accumulate into grad_value ---

@pytest.mark.parametrize("dtype,C_h", [("fp32", 32), ("fp32", 6), ("bf16", 32), ("bf16", 6)])
def test_accumulate_grad_value(dtype, C_h, gpu_device):
    """grad_value += result: the old contents plus the oracle's gradient (both
    the tiled path, C_h = 32, and the generic one, C_h = 6)."""
    import torch
    from scale_deformable_attention_forward_amd import msda_backward
    d = _mk(seed=23, C_h=C_h, N_q=400, N_h=2, levels=((12, 14), (3, 4)), value_dtype=dtype)
    t = to_device(d, gpu_device)
    rng = np.random.default_rng(99)
    init = rng.standard_normal(t["value"].shape).astype(np.float32)
    gv = torch.from_numpy(init).to(gpu_device).to(t["value"].dtype)
    init_used = to_numpy(gv).astype(np.float64)        # exact bf16 values when bf16
    res = msda_backward(t["grad_output"], t["value"], d["spatial_shapes"], d["level_start_index"],
                        t["sampling_locations"], t["attention_weights"], grad_value=gv,
                        accumulate_grad_value=True)
    torch.cuda.synchronize()
    assert res[0] is gv
    want = oracle_backward(d)
    compare(f"accumulated grad_value {dtype} C_h={C_h}", to_numpy(gv), init_used + want[0], RTOL[dtype])
    compare(f"grad_loc with accumulate {dtype}", to_numpy(res[1]), want[1], RTOL[dtype])


def test_accumulate_twice_equals_double(gpu_device):
    """Two accumulating calls from zero give twice one call's gradient (the
    chunked backward use: the same buffer collects several calls)."""
    import torch
    from scale_deformable_attention_forward_amd import msda_backward
    d = _mk(seed=25, C_h=32, N_q=500, N_h=2)
    t = to_device(d, gpu_device)
    gv = torch.zeros_like(t["value"])
    for _ in range(2):
        msda_backward(t["grad_output"], t["value"], d["spatial_shapes"], d["level_start_index"],
                      t["sampling_locations"], t["attention_weights"], grad_value=gv,
                      compute_grad_sampling_locations=False, compute_grad_attention_weights=False,
                      accumulate_grad_value=True)
    torch.cuda.synchronize()
    want = oracle_backward(d, compute_grad_sampling_locations=False, compute_grad_attention_weights=False)[0]
    compare("two accumulating calls", to_numpy(gv), 2.0 * want, RTOL["fp32"])


def test_empty_problem_accumulate_leaves_grad_value(gpu_device):
    import torch
    from scale_deformable_attention_forward_amd import msda_backward
    d = _mk(seed=26, N_q=0)
    t = to_device(d, gpu_device)
    gv = torch.full_like(t["value"], 3.0)
    msda_backward(t["grad_output"], t["value"], d["spatial_shapes"], d["level_start_index"],
                  t["sampling_locations"], t["attention_weights"], grad_value=gv, accumulate_grad_value=True)
    torch.cuda.synchronize()
    assert bool((gv == 3.0).all().item())


def test_unaligned_bf16_backward_takes_generic_path(gpu_device):
    """A grad_value view one element into its allocation cannot take the tiled
    path's 8-byte accesses; the generic path must give the same result."""
    import torch
    from scale_deformable_attention_forward_amd import msda_backward
    d = _mk(seed=27, C_h=8, value_dtype="bf16")
    t = to_device(d, gpu_device)
    buf = torch.empty(t["value"].numel() + 1, dtype=torch.bfloat16, device=gpu_device)
    gv = buf[1:].view(t["value"].shape)
    res = msda_backward(t["grad_output"], t["value"], d["spatial_shapes"], d["level_start_index"],
                        t["sampling_locations"], t["attention_weights"], grad_value=gv)
    torch.cuda.synchronize()
    want = oracle_backward(d)
    for n, g, w in zip(("grad_value", "grad_loc", "grad_attn"), res, want):
        compare(f"unaligned bf16 {n}", to_numpy(g), w, RTOL["bf16"])


def test_bf16_rows_off_16_bytes_gather_four_channels_a_lane(gpu_device):
    """value and grad_output views 8 bytes (four bfloat16 elements) into their
    allocations: the tiled path still applies, but its gather of grad_A and
    grad_loc takes 4 channels a lane instead of 8."""
    import torch
    from scale_deformable_attention_forward_amd import msda_backward
    d = _mk(seed=59, C_h=32, N_q=200, N_h=4, value_dtype="bf16")
    t = to_device(d, gpu_device)
    views = {}
    for name in ("value", "grad_output"):
        x = t[name]
        buf = torch.empty(x.numel() + 4, dtype=x.dtype, device=gpu_device)
        views[name] = buf[4:].view(x.shape)
        views[name].copy_(x)
        assert views[name].data_ptr() % 16 == 8
    res = msda_backward(views["grad_output"], views["value"], d["spatial_shapes"], d["level_start_index"],
                        t["sampling_locations"], t["attention_weights"])
    torch.cuda.synchronize()
    want = oracle_backward(d)
    for n, g, w in zip(("grad_value", "grad_loc", "grad_attn"), res, want):
        compare(f"bf16 rows off 16 bytes {n}", to_numpy(g), w, RTOL["bf16"])
