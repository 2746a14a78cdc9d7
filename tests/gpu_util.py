"""Shared helpers of the GPU tests: seeded inputs in both precisions and the parity measure."""
from __future__ import annotations

import numpy as np

import gdn_synth

TOL = {"f32": 1e-4, "bf16": 1e-2}   # max|d| / max|ref|, fp32 state in both cases


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite GPU values"
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def random_qkv(rng, shape, dtype, relu=False):
    """fp32 values already representable in `dtype` (bf16 rounding done on the host)."""
    out = []
    for i in range(3):
        x = rng.standard_normal(shape).astype(np.float32)
        if relu and i < 2:
            x = np.maximum(x, 0)
        if dtype == "bf16":
            x = gdn_synth.bf16_bits_to_f32(gdn_synth.f32_to_bf16_bits(x))
        out.append(x)
    return out


def to_dev(x, dtype, dev, layout="head"):
    """[B, H, T, D] fp32 numpy -> torch tensor of `dtype` with the given storage layout."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    if layout == "token":
        t = t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    return t.to(dev)


def to_np(t):
    return t.float().cpu().numpy()
