"""Helpers for GPU parity tests: move seeded inputs to the device, run the
kernel through the C ABI, compare with the float64 oracle."""
from __future__ import annotations

import sys

import numpy as np

# O tolerances are the ones the target states for bf16 inputs; the lse bound
# is derived from the arithmetic (scores and sums in float32 from exact bf16
# products: errors ~1e-6), with a wide margin.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(case, dev="cuda:0"):
    import torch
    t = {n: torch.from_numpy(np.ascontiguousarray(case[n]).view(np.int16)).view(torch.bfloat16).to(dev)
         for n in ("q", "k", "v")}
    kpm = None if case["kpm"] is None else torch.from_numpy(np.ascontiguousarray(case["kpm"])).to(dev)
    return t["q"], t["k"], t["v"], kpm


def run_gpu(case, dev="cuda:0"):
    import torch

    import exact_attention_44_amd as E
    q, k, v, kpm = to_device(case, dev)
    out, lse = E.fwd(q, k, v, causal=bool(case["causal"]), key_padding_mask=kpm,
                     scale=float(case["scale"]))
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def f64(case, n):
    from workloads import bf16_bits_to_f32
    return bf16_bits_to_f32(case[n]).astype(np.float64)


def compare(O, lse, O_ref, lse_ref, what=""):
    """Element-wise parity of O and lse; returns (max|dO|, mean|dO|, max|dlse|)."""
    assert O.shape == O_ref.shape and lse.shape == lse_ref.shape
    assert np.all(np.isfinite(O)), f"{what}: non-finite output"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf lse pattern differs"
    assert np.all(O[empty] == 0.0), f"{what}: rows with no visible key must be zero"
    err = np.abs(O - O_ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    lerr = float(np.max(np.abs(lse[~empty] - lse_ref[~empty]))) if (~empty).any() else 0.0
    say(f"  {what}: max|dO|={mx:.3e} mean|dO|={mean:.3e} max|dlse|={lerr:.3e}")
    assert mx <= O_MAX_ABS, f"{what}: max|dO| {mx} > {O_MAX_ABS}"
    assert mean <= O_MEAN_ABS, f"{what}: mean|dO| {mean} > {O_MEAN_ABS}"
    assert lerr <= LSE_MAX_ABS, f"{what}: max|dlse| {lerr} > {LSE_MAX_ABS}"
    return mx, mean, lerr
