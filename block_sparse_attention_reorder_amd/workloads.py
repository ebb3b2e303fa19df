"""The synthetic workloads: token grid, tile shape, heads, head size and input recipe.

Shapes follow the models the pages evaluate on (Wan2.1-1.3B and -14B at 480p/720p,
HunyuanVideo at 720p, a Flux-sized 8192x8192 image) [FPSAttention: Training-Aware
FP8 and Sparsity Co-Design for Fast Video Diffusion, Abstract] [LoSA: Near-Lossless
Sparse Attention for Training-Free Video Diffusion Acceleration, Abstract] [Grouping
First, Attending Smartly: Training-Free Acceleration for Diffusion Transformers,
Abstract]. Video latents use 4x4x4 token tiles (64 tokens); the image uses 8x8
token groups. No arithmetic of the method lives here.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    grid: tuple            # (T, H, W) unpadded token grid; T = 1 for an image
    tile: tuple            # (tt, th, tw), product 64
    B: int
    H: int
    D: int
    dtype: str             # "f32" or "bf16": precision of the generated Q/K/V
    amp: float             # weight of the positional signal
    sigma: float           # noise std for step 0
    seed: int
    reuse_steps: int = 0   # later calls that reuse the step-0 block selection
    fp8: bool = False      # also run the FP8 e4m3 Q/K forward
    mask: str = "mass"     # "mass": mass pass + 99 % selection; "grat": fixed structured mask
    note: str = ""

    @property
    def N(self) -> int:
        T, Hg, Wg = self.grid
        return T * Hg * Wg

    def sigma_at(self, step: int) -> float:
        """Noise std of call ``step`` (0 = the dense selection step)."""
        return self.sigma if step == 0 else 0.9 ** step


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", (4, 8, 8), (4, 4, 4), 1, 1, 64, "f32", 0.5, 1.0, 0,
                 note="256 tokens, 4 blocks; float32 inputs"),
        Workload("wan480p", (21, 30, 52), (4, 4, 4), 1, 12, 128, "bf16", 1.0, 1.0, 0,
                 note="Wan2.1-1.3B-shaped 480p latent, 32,760 tokens"),
        Workload("wan720p", (21, 45, 80), (4, 4, 4), 1, 40, 128, "bf16", 1.0, 1.0, 0, fp8=True,
                 note="Wan2.1-14B-shaped 720p latent, 75,600 tokens; bf16 and FP8 Q/K"),
        Workload("hunyuan720p", (33, 45, 80), (4, 4, 4), 1, 24, 128, "bf16", 1.5, 1.0, 0, reuse_steps=10,
                 note="HunyuanVideo-shaped 720p latent, 118,800 tokens; 10 frozen-mask calls"),
        Workload("grat8192", (1, 512, 512), (1, 8, 8), 1, 24, 128, "bf16", 1.0, 1.0, 0, mask="grat",
                 note="Flux-shaped 8192x8192 image, 262,144 tokens; fixed structured mask"),
    ]
}
