"""Seeded synthetic inputs for the sparse-linear attention workloads.

This module draws the operands only: Q, K, V, the projection weight W and the
output gradient dO, as bf16 bit patterns (numpy ``uint16``).  It holds no step
of the attention method itself, so both the CPU oracle (through the tests) and
the GPU library can consume the very same bits.

Recipe (a stand-in for DiT activations, which are not available here):

* tokens sit on a video (T, H, W) or image (H, W) grid in raster order, last
  axis fastest;
* each grid axis of length L contributes four low-frequency features of the
  coordinate p: sin(pi p / L), cos(pi p / L), sin(2 pi p / L), cos(2 pi p / L);
* per head h a Gaussian matrix G_h (entries of variance 1/F, F = 4 * axes)
  projects the features to d dimensions; the same G_h is used for Q and K of
  every batch item, so q . k peaks for tokens that are close on the grid;
* Q = feat G_h + noise, K = feat G_h + noise, noise of variance 0.5;
  V ~ N(0, 1); W ~ N(0, 1/d) as a d x d matrix; dO ~ N(0, 1);
* tokens past ``valid_len`` are padding and are all-zero.

Draw order from one numpy PCG64 stream: all G_h; then per batch item the Q
noise, the K noise and V (each [H, valid_len, d], float32 draws); then W;
then dO (float32 draws, padded rows zero).  Values are rounded to bf16 with
round-to-nearest-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

BLOCK = 64


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    grid: tuple
    valid_len: int
    frac_critical: float
    frac_negligible: float

    @property
    def num_blocks(self) -> int:
        return self.seq_len // BLOCK


# The five workloads of the method's evaluation set-up, named by what they are.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("video_tiny_b1_h2_n1024_d64", 1, 2, 1024, 64, (8, 8, 16), 1024, 0.125, 0.25),
        Workload("video_b1_h12_n8192_d128", 1, 12, 8192, 128, (8, 32, 32), 8192, 0.05, 0.10),
        Workload("video_dit_b2_h12_n32768_d128", 2, 12, 32768, 128, (21, 30, 52), 32760, 0.05, 0.10),
        Workload("pixel_b1_h8_n65536_d64", 1, 8, 65536, 64, (256, 256), 65536, 0.02, 0.20),
        Workload("video_bwd_b1_h12_n16384_d128", 1, 12, 16384, 128, (16, 32, 32), 16384, 0.05, 0.10),
    )
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def grid_features(grid: tuple, count: int) -> np.ndarray:
    """[count, 4 * len(grid)] float64 features of the first ``count`` grid tokens."""
    n = np.arange(count)
    coords = np.unravel_index(n, grid)
    cols = []
    for p, length in zip(coords, grid):
        p = p.astype(np.float64)
        for f in (1.0, 2.0):
            cols.append(np.sin(f * math.pi * p / length))
            cols.append(np.cos(f * math.pi * p / length))
    return np.stack(cols, axis=1)


def make_inputs(batch: int, heads: int, seq_len: int, head_dim: int, grid: tuple,
                valid_len: int | None = None, seed: int = 0, with_grad: bool = True) -> dict:
    """Draw one problem.  Returns uint16 bf16 bit arrays q, k, v, do [B,H,N,d]
    and w [d,d], plus the seed and valid_len."""
    if valid_len is None:
        valid_len = seq_len
    if not (0 < valid_len <= seq_len):
        raise ValueError("valid_len must be in (0, seq_len]")
    if valid_len > int(np.prod(grid)):
        raise ValueError("grid holds fewer tokens than valid_len")
    rng = np.random.Generator(np.random.PCG64(seed))
    nfeat = 4 * len(grid)
    feat = grid_features(grid, valid_len)
    proj = rng.standard_normal((heads, nfeat, head_dim)) * math.sqrt(1.0 / nfeat)
    noise_std = np.float32(math.sqrt(0.5))
    shape = (batch, heads, seq_len, head_dim)
    q = np.zeros(shape, np.uint16)
    k = np.zeros(shape, np.uint16)
    v = np.zeros(shape, np.uint16)
    base = [(feat @ proj[h]).astype(np.float32) for h in range(heads)]
    for b in range(batch):
        eq = rng.standard_normal((heads, valid_len, head_dim), dtype=np.float32) * noise_std
        ek = rng.standard_normal((heads, valid_len, head_dim), dtype=np.float32) * noise_std
        vv = rng.standard_normal((heads, valid_len, head_dim), dtype=np.float32)
        for h in range(heads):
            q[b, h, :valid_len] = f32_to_bf16_bits(base[h] + eq[h])
            k[b, h, :valid_len] = f32_to_bf16_bits(base[h] + ek[h])
        v[b, :, :valid_len] = f32_to_bf16_bits(vv)
        del eq, ek, vv
    w = f32_to_bf16_bits(rng.standard_normal((head_dim, head_dim), dtype=np.float32)
                         * np.float32(math.sqrt(1.0 / head_dim)))
    out = dict(q=q, k=k, v=v, w=w, valid_len=valid_len, seed=seed)
    if with_grad:
        do = np.zeros(shape, np.uint16)
        for b in range(batch):
            do[b, :, :valid_len] = f32_to_bf16_bits(
                rng.standard_normal((heads, valid_len, head_dim), dtype=np.float32))
        out["do"] = do
    return out


def make_workload_inputs(name: str, seed: int = 0, with_grad: bool = True) -> dict:
    w = WORKLOADS[name]
    return make_inputs(w.batch, w.heads, w.seq_len, w.head_dim, w.grid, w.valid_len,
                       seed=seed, with_grad=with_grad)


def random_bf16(shape, seed: int, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """Plain i.i.d. Gaussian bf16 bits, for edge-case tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(std) + np.float32(mean)
    return f32_to_bf16_bits(x)
