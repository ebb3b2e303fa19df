"""Seeded synthetic inputs shared by the HIP path and the CPU oracle.

This module only draws inputs; it holds none of the method's arithmetic (no tiling,
no attention, no block masses, no selection). Both sides consume exactly the arrays
produced here.

The pages measure on trained video and image diffusion transformers (Wan2.1,
HunyuanVideo, Flux) whose activations are not available; the stand-in is a
sinusoidal positional signal over the token grid plus Gaussian noise, which gives
attention the local structure that block selection exploits
[LoSA: Near-Lossless Sparse Attention for Training-Free Video Diffusion
Acceleration, Abstract] [Grouping First, Attending Smartly: Training-Free
Acceleration for Diffusion Transformers, Abstract].

Recipe (all configs, batch B):
  * tokens are listed in raster order over the unpadded grid (t slowest, w fastest);
    a 2D image is a grid with T = 1;
  * pe[n, 2i] = sin(w_i * pos_a(i)(n)), pe[n, 2i+1] = cos(w_i * pos_a(i)(n)) with
    w_i = 10000 ** (-2 i / D) and a(i) = i mod 3 over (t, h, w), or i mod 2 over
    (h, w) for a 2D grid; evaluated in float64, then cast to float32;
  * noise = numpy default_rng(seed).standard_normal((3, B, N, H, D), float32),
    slices 0, 1, 2 give Q, K, V in [B, N, H, D] raster layout;
  * x = float32(amp) * pe + float32(sigma) * noise, as a float32 multiply then a
    float32 add (numpy evaluates these elementwise with no fused multiply-add);
  * bf16 workloads round x to bfloat16 (round to nearest even); both sides then
    use those bfloat16 values (the oracle upcasts them to float32 exactly).
"""
from __future__ import annotations

import numpy as np

__all__ = ["positional_features", "make_qkv", "to_bf16_values", "random_mass_rows"]


def positional_features(grid: tuple[int, int, int], D: int) -> np.ndarray:
    """Sinusoidal features [N, D] float32 for the raster tokens of an unpadded grid."""
    T, Hg, Wg = grid
    if D % 2:
        raise ValueError("D must be even")
    t, h, w = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(Wg), indexing="ij")
    axes3 = [t.reshape(-1).astype(np.float64), h.reshape(-1).astype(np.float64), w.reshape(-1).astype(np.float64)]
    axes = axes3 if T > 1 else axes3[1:]
    N = T * Hg * Wg
    pe = np.empty((N, D), dtype=np.float64)
    for i in range(D // 2):
        omega = 10000.0 ** (-2.0 * i / D)
        pos = axes[i % len(axes)]
        pe[:, 2 * i] = np.sin(omega * pos)
        pe[:, 2 * i + 1] = np.cos(omega * pos)
    return pe.astype(np.float32)


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even) and return them as float32."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def make_qkv(grid, B: int, H: int, D: int, amp: float, sigma: float, seed: int,
             bf16: bool = True):
    """Q, K, V in raster layout [B, N, H, D] float32 (bf16-rounded when ``bf16``)."""
    T, Hg, Wg = grid
    N = T * Hg * Wg
    pe = positional_features(grid, D)                      # [N, D]
    rng = np.random.default_rng(seed)
    noise = rng.standard_normal((3, B, N, H, D), dtype=np.float32)
    a = np.float32(amp)
    s = np.float32(sigma)
    base = (a * pe).astype(np.float32)[None, :, None, :]   # [1, N, 1, D]
    out = []
    for idx in range(3):
        x = np.multiply(s, noise[idx], dtype=np.float32)
        np.add(base, x, out=x, dtype=np.float32)
        out.append(to_bf16_values(x) if bf16 else x)
    del noise
    return out[0], out[1], out[2]


def random_mass_rows(R: int, nb: int, seed: int, tie_frac: float = 0.1,
                     zero_frac: float = 0.05) -> np.ndarray:
    """Seeded non-negative float32 rows [R, nb] standing in for block masses.

    Heavy-tailed magnitudes, a fraction of exact duplicates (ties) and exact zeros,
    each row scaled to sum to about one, so that selection sees the same kinds of
    rows the mass pass produces and also the awkward ones (ties, zeros, spikes).
    """
    rng = np.random.default_rng(seed)
    x = rng.exponential(1.0, size=(R, nb)) ** 3
    ties = rng.random((R, nb)) < tie_frac
    src = rng.integers(0, nb, size=(R, nb))
    rows = np.arange(R)[:, None]
    x = np.where(ties, x[rows, src], x)
    x = np.where(rng.random((R, nb)) < zero_frac, 0.0, x)
    ssum = x.sum(axis=1, keepdims=True)
    ssum[ssum == 0] = 1.0
    return (x / ssum).astype(np.float32)
