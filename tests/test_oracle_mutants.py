"""The pins must be able to fail: plant plausible mistakes in a copy of the
oracle's C source (on the CPU), rebuild it, and check that at least one pin
rejects every mutant. The committed oracle is never modified."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import bruteforce

import test_oracle_pins as pins  # noqa: E402

SRC = os.path.join(os.path.dirname(oracle.__file__), "msda_oracle.c")

MUTANTS = {
    "x_y_swapped": ("double x = pixel_coord(P, lx, W, &K->sx);", "double x = pixel_coord(P, ly, W, &K->sx);"),
    "column_major_level": ("K->pix[k] = start + yi * W + xi;", "K->pix[k] = start + xi * H + yi;"),
    "dwdx_sign": ("K->dwdx[k] = (dx ? 1.0 : -1.0) * wy;", "K->dwdx[k] = (dx ? -1.0 : 1.0) * wy;"),
    "half_pixel_dropped": ("fmaf(lf, (float)size, -0.5f)", "fmaf(lf, (float)size, 0.0f)"),
    "slope_off_by_one": ("*slope = P->align_corners ? (double)(size - 1) : (double)size;",
                         "*slope = (double)(size - 1);"),
    "border_clamp_keeps_slope": ("if (x < 0.0) { x = 0.0; *slope = 0.0; }", "if (x < 0.0) { x = 0.0; }"),
    "blnc_head_pixel_swapped": ("return ((b * P->L + pix) * P->Nh + h) * P->Ch + c;",
                                "return ((b * P->Nh + h) * P->L + pix) * P->Ch + c;"),
    "corner_weight_transposed": ("K->w[k] = wx * wy;", "K->w[k] = dx == dy ? wx * wy : (1.0 - wx) * (1.0 - wy);"),
    "grad_value_missing_weight": ("+= a * K.w[k] * g[c];", "+= a * g[c];"),
    "upper_bound_inclusive": ("K->inb[k] = (xi >= 0 && xi < W && yi >= 0 && yi < H);",
                              "K->inb[k] = (xi >= 0 && xi <= W && yi >= 0 && yi < H);"),
}


def _pins_pass():
    """A compact run of the pins that exercise every line of the oracle."""
    try:
        pins.test_hand_worked_golden_forward()
        pins.test_hand_worked_golden_backward()
        for mode in pins.MODES:
            pins.test_matches_grid_sample_composition(mode)
        for align in (False, True):
            for pad in ("zeros", "border"):
                pins.test_central_finite_differences(align, pad)
        return True
    except AssertionError:
        return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, tmp_path):
    pytest.importorskip("torch")
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-o", str(so),
                    str(mut), "-lm"], check=True)
    saved = oracle._load()
    try:
        oracle._lib = oracle.bind(str(so))
        assert not _pins_pass(), f"no pin caught mutant {name}"
    finally:
        oracle._lib = saved
    assert _pins_pass()
