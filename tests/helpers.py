"""Shared helpers of the test suite: device upload of seeded inputs, the oracle
call on the same inputs, and the comparison rule.

Comparison rule (the reading of "1e-5 relative (fp32) or 2e-2 (bf16 value,
fp32 accumulate)"): every element must satisfy
    |gpu - oracle| <= rtol * (|oracle| + rms(oracle))
with rms over the whole tensor, so that outputs near zero and the last-bit
noise of float32 atomics are judged against the tensor's scale.

Where one element sums thousands of terms that cancel (thousands of samples
piled onto one pixel), the rounding error of any float32 summation grows
with the sum of the terms' magnitudes, not with the result: tests of such
inputs pass that sum (the oracle's grad_value for |grad_output| and |A|,
the bilinear weights being non-negative) as ``magnitude``, which joins the
scale. A single wrong or missing term still exceeds rtol times it as long
as an element has fewer than 1 / rtol terms.
"""
import numpy as np

import oracle

RTOL = {"fp32": 1e-5, "bf16": 2e-2}


def to_device(d, device):
    import torch
    out = {}
    if d["value_dtype"] == "bf16":
        bits = d["value_bf16_bits"]
        out["value"] = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(device)
    else:
        out["value"] = torch.from_numpy(d["value"]).to(device)
    out["sampling_locations"] = torch.from_numpy(d["sampling_locations"]).to(device)
    out["attention_weights"] = torch.from_numpy(d["attention_weights"]).to(device)
    if "grad_output" in d:
        g = torch.from_numpy(d["grad_output"]).to(device)
        out["grad_output"] = g.to(torch.bfloat16) if d["value_dtype"] == "bf16" else g
    return out


def to_numpy(t):
    import torch
    if t is None:
        return None
    return t.detach().to(torch.float32).cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def oracle_forward(d, **over):
    args = dict(value=d["value"], spatial_shapes=d["spatial_shapes"],
                level_start_index=d["level_start_index"], sampling_locations=d["sampling_locations"],
                attention_weights=d["attention_weights"], value_layout=d["value_layout"],
                sampling_locations_layout=d["sampling_locations_layout"],
                align_corners=d["align_corners"], padding_mode=d["padding_mode"])
    args.update(over)
    return oracle.forward(**args)


def oracle_backward(d, **over):
    args = dict(grad_output=d["grad_output"], value=d["value"], spatial_shapes=d["spatial_shapes"],
                level_start_index=d["level_start_index"], sampling_locations=d["sampling_locations"],
                attention_weights=d["attention_weights"], value_layout=d["value_layout"],
                sampling_locations_layout=d["sampling_locations_layout"],
                align_corners=d["align_corners"], padding_mode=d["padding_mode"])
    args.update(over)
    return oracle.backward(**args)


def compare(name, got, want, rtol, magnitude=None):
    """Assert the comparison rule; returns (max |err| / scale, worst index).
    ``magnitude`` (per element, same shape) joins the scale where elements
    are sums of many cancelling terms."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{name}: shape {got.shape} != {want.shape}"
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    if want.size == 0:
        return 0.0, None
    rms = float(np.sqrt(np.mean(want * want)))
    scale = np.abs(want) + rms
    if magnitude is not None:
        magnitude = np.asarray(magnitude, dtype=np.float64)
        assert magnitude.shape == want.shape and (magnitude >= 0).all(), f"{name}: bad magnitude"
        scale = scale + magnitude
    scale = np.where(scale > 0, scale, 1.0)
    rel = np.abs(got - want) / scale
    worst = np.unravel_index(int(np.argmax(rel)), rel.shape)
    err = float(rel[worst])
    assert err <= rtol, (f"{name}: max err {err:.3e} > {rtol:.1e} at {worst}: "
                         f"gpu {got[worst]!r} oracle {want[worst]!r} (rms {rms:.3e})")
    return err, worst
