"""Shared test plumbing: stored arrays -> device tensors, and the comparison bar."""
from __future__ import annotations

import numpy as np

TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 2e-2)}   # (atol, rtol) per storage dtype


def to_device(arr, device="cuda"):
    import torch
    if arr.dtype == np.uint16:   # bf16 bit patterns
        return torch.from_numpy(arr.view(np.int16).copy()).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def to_f64(t):
    """Device tensor -> float64 numpy, exactly."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy().astype(np.float64)


def compare(got, ref, dtype, what=""):
    """|got - ref| <= atol + rtol |ref| elementwise; NaN/Inf fail. Returns the max abs error."""
    atol, rtol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{bad.size} elements off; max abs err {err.max():.3e}, "
                           f"first at {np.argwhere(bad)[0].tolist()}")
    return float(err.max())
