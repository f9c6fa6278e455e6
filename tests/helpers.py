"""Shared helpers for the GPU parity tests (comparison metrics, runners)."""
from __future__ import annotations

import os
import sys

import numpy as np

import oracle as orc

# Output tolerance of the method: bf16 inputs, fp32 accumulation.
REL_L2 = 1e-2
MAX_ABS = 2e-2


def ensure_library():
    from sparse_linear_attention_mean_amd import builder

    if not os.path.exists(builder.LIB):
        builder.build()


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.sqrt((b * b).sum())
    num = np.sqrt(((a - b) ** 2).sum())
    return float(num / den) if den > 0 else float(num)


def assert_close(name, got, ref, rel=REL_L2, atol=MAX_ABS):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    r = rel_l2(got, ref)
    m = float(np.abs(got - ref).max()) if got.size else 0.0
    print(f"  {name}: rel_l2={r:.3e} max_abs={m:.3e}", flush=True)
    assert r <= rel, f"{name}: rel-L2 {r:.3e} > {rel}"
    assert m <= atol, f"{name}: max-abs {m:.3e} > {atol}"


def to_np(t):
    import torch

    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def device_inputs(inp, device="cuda"):
    from sparse_linear_attention_mean_amd.attention import bf16_from_bits

    out = {k: bf16_from_bits(inp[k], device) for k in ("q", "k", "v", "w")}
    if "do" in inp:
        out["do"] = bf16_from_bits(inp["do"], device)
    return out


def decoded(inp):
    return {k: orc.decode_bf16(inp[k]) for k in ("q", "k", "v", "w", "do") if k in inp}


def mask_validity(gpu_mask, scores, k_c, k_n, tol):
    """Check that a GPU mask is a correct classification of the oracle's fp32
    scores up to ``tol`` (the rounding gap between independently computed
    score maps).  Returns the boolean [.., T] array of rows equal to the
    oracle's own classification."""
    ref = orc.classify(scores, k_c, k_n)
    same = (gpu_mask == ref).all(axis=-1)
    flat_g = gpu_mask.reshape(-1, gpu_mask.shape[-1])
    flat_s = scores.reshape(-1, scores.shape[-1]).astype(np.float64)
    for r in np.flatnonzero(~same.reshape(-1)):
        g, s = flat_g[r], flat_s[r]
        assert (g == 1).sum() == k_c and (g == -1).sum() == k_n, "row counts"
        crit, marg, negl = s[g == 1], s[g == 0], s[g == -1]
        if crit.size and marg.size:
            assert crit.min() >= marg.max() - tol, "critical/marginal order beyond rounding"
        if marg.size and negl.size:
            assert marg.min() >= negl.max() - tol, "marginal/negligible order beyond rounding"
        if crit.size and negl.size and not marg.size:
            assert crit.min() >= negl.max() - tol
    return same


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()
