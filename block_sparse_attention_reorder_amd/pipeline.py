"""The whole hot path on one GPU, as calls into libfpsa.

    raster Q, K, V --tile--> tiled Q, K (QK operand layout) and V (VT)
        --block_mass--> M[B, H, nb, nb] --select_blocks (99 %)--> frozen CSR
        --sparse_attn_fwd--> tiled O --tile (inverse)--> raster O

The measurement and selection happen once; the CSR is then reused for every later
call [LoSA: Near-Lossless Sparse Attention for Training-Free Video Diffusion
Acceleration, Abstract]. A fixed structured CSR can stand in for the measured one
[Grouping First, Attending Smartly: Training-Free Acceleration for Diffusion
Transformers, Abstract], and so can fixed per-head diagonal / multi-diagonal /
stripe patterns [Sparse-vDiT: Unleashing the Power of Sparse Attention to Accelerate
Video Diffusion Transformers, Abstract]; `retained_mass` reports how much of a
later step's mass the frozen CSR still covers. This module only allocates device buffers (torch) and
sequences the library calls; all arithmetic runs in the HIP kernels.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import fpsa


@dataclass
class Csr:
    row_ptr: torch.Tensor      # int32 [R + 1]
    col_idx: torch.Tensor      # int32 [capacity]; the first row_ptr[R] entries are used

    def nnz(self) -> int:
        return int(self.row_ptr[-1].item())


class BlockSparseAttention:
    """Buffers and calls for one geometry (grid, tile, B, H, D) on one device."""

    def __init__(self, grid, tile, B, H, D, device="cuda", softmax_scale=None):
        self.grid, self.tile = tuple(grid), tuple(tile)
        self.B, self.H, self.D = int(B), int(H), int(D)
        self.device = torch.device(device)
        self.nb = fpsa.num_blocks(self.grid, self.tile)
        if self.nb <= 0:
            raise ValueError(f"invalid grid {grid} / tile {tile}")
        self.N = self.grid[0] * self.grid[1] * self.grid[2]
        self.npad = 64 * self.nb
        self.R = self.B * self.H * self.nb
        self.scale = float(softmax_scale) if softmax_scale is not None else 1.0 / math.sqrt(self.D)

    # ------------------------------------------------------------------ layout
    def tiled_shape(self):
        return (self.B, self.H, self.npad, self.D)

    def tile_rows(self, x, out=None, stream=None):
        """raster [B, N, H, D] (f32/bf16) -> tiled rows bf16."""
        out = torch.empty(self.tiled_shape(), dtype=torch.bfloat16, device=self.device) if out is None else out
        fpsa.tile_reorder(x, out, self.grid, self.tile, self.B, self.H, self.D, stream=stream)
        return out

    def tile_qk(self, x, out=None, stream=None):
        """raster [B, N, H, D] (f32/bf16) -> tiled QK operand layout bf16 (for Q and K)."""
        out = torch.empty(self.tiled_shape(), dtype=torch.bfloat16, device=self.device) if out is None else out
        fpsa.tile_reorder(x, out, self.grid, self.tile, self.B, self.H, self.D, layout=fpsa.LAYOUT_QK,
                          stream=stream)
        return out

    def tile_vt(self, x, out=None, stream=None):
        """raster [B, N, H, D] -> tiled VT bf16 (value operand layout)."""
        out = torch.empty(self.tiled_shape(), dtype=torch.bfloat16, device=self.device) if out is None else out
        fpsa.tile_reorder(x, out, self.grid, self.tile, self.B, self.H, self.D, layout=fpsa.LAYOUT_VT,
                          stream=stream)
        return out

    def tile_fp8(self, x, out=None, scale=None, layout=fpsa.LAYOUT_QK, stream=None):
        """raster [B, N, H, D] -> tiled e4m3 bytes (QK layout by default) + per-tile
        float32 scales [B, H, nb]."""
        out = torch.empty(self.tiled_shape(), dtype=torch.uint8, device=self.device) if out is None else out
        scale = torch.empty((self.B, self.H, self.nb), dtype=torch.float32, device=self.device) if scale is None else scale
        fpsa.tile_reorder(x, out, self.grid, self.tile, self.B, self.H, self.D, layout=layout, dst_scale=scale,
                          stream=stream)
        return out, scale

    def dequantize(self, x8, scale, out=None, stream=None):
        """e4m3 QK tiles and their per-tile scales -> bf16 QK tiles of the dequantized
        values; scale None gives the code values themselves (the operands of the FP8
        forward's backward, which takes the scales separately)."""
        out = torch.empty(self.tiled_shape(), dtype=torch.bfloat16, device=self.device) if out is None else out
        fpsa.dequantize_tiles(x8, scale, self.grid, self.tile, self.B, self.H, self.D, out, stream=stream)
        return out

    def untile(self, o_tiled, dtype=torch.bfloat16, out=None, stream=None):
        """tiled rows bf16 -> raster [B, N, H, D] of dtype (real tokens only)."""
        out = torch.empty((self.B, self.N, self.H, self.D), dtype=dtype, device=self.device) if out is None else out
        fpsa.tile_reorder(o_tiled, out, self.grid, self.tile, self.B, self.H, self.D, inverse=True, stream=stream)
        return out

    # ------------------------------------------------------------------ selection
    # Default bound on the mass pass's scratch: the per-query-block log-sum-exps of the
    # query blocks in flight (nb * 64 * 4 bytes each). The whole grid's would be 28.7 GB
    # at the HunyuanVideo shape; 2 GiB holds two waves of workgroups there, and the pass
    # runs in several launches of whole waves.
    MASS_WORKSPACE_CAP = 2 << 30

    def mass_workspace(self, max_bytes=MASS_WORKSPACE_CAP):
        """Scratch for the mass pass: enough for one launch, or at most max_bytes
        (then the pass runs in several launches); max_bytes=None takes the whole grid."""
        n = fpsa.mass_workspace_bytes(self.B, self.H, self.grid, self.tile)
        if max_bytes is not None:
            n = max(min(n, int(max_bytes)), 2 * self.nb * 64 * 4)
        return torch.empty(n, dtype=torch.uint8, device=self.device)

    def block_mass(self, qt, kt, mass=None, lse=None, want_lse=False, workspace=None, stream=None):
        mass = torch.empty((self.B, self.H, self.nb, self.nb), dtype=torch.float32, device=self.device) if mass is None else mass
        if want_lse and lse is None:
            lse = torch.empty((self.B, self.H, self.npad), dtype=torch.float32, device=self.device)
        ws = self.mass_workspace() if workspace is None else workspace
        fpsa.block_mass(qt, kt, self.grid, self.tile, self.B, self.H, self.D, self.scale, mass, ws, lse,
                        stream=stream)
        return (mass, lse) if want_lse else mass

    def new_csr(self, capacity=None) -> Csr:
        cap = self.R * self.nb if capacity is None else int(capacity)
        return Csr(torch.empty(self.R + 1, dtype=torch.int32, device=self.device),
                   torch.empty(cap, dtype=torch.int32, device=self.device))

    def workspace(self, rows=None):
        n = fpsa.select_workspace_bytes(self.R if rows is None else rows, self.nb)
        return torch.empty(max(n, 1), dtype=torch.uint8, device=self.device)

    def select(self, mass, thr_num=99, thr_den=100, csr=None, workspace=None, stream=None) -> Csr:
        csr = self.new_csr() if csr is None else csr
        ws = self.workspace() if workspace is None else workspace
        fpsa.select_blocks(mass, self.R, self.nb, thr_num, thr_den, csr.row_ptr, csr.col_idx, ws, stream=stream)
        return csr

    def structured(self, stream=None) -> Csr:
        nh = -(-self.grid[1] // self.tile[1])
        nw = -(-self.grid[2] // self.tile[2])
        csr = self.new_csr(capacity=self.R * (nh + nw + 9))
        ws = self.workspace()
        fpsa.structured_mask(self.grid, self.tile, self.B * self.H, csr.row_ptr, csr.col_idx, ws, stream=stream)
        return csr

    def frame_period(self) -> int:
        """Blocks per tile-grid time slice (nh * nw): the block offset between a
        tile and the tile at the same spatial place one time slice later, the
        natural period of a multi-diagonal pattern on video grids."""
        return (-(-self.grid[1] // self.tile[1])) * (-(-self.grid[2] // self.tile[2]))

    def pattern(self, patterns, stream=None) -> Csr:
        """CSR of fixed per-head patterns: H tuples (band, period, stripe, dense)
        or an int32 [H, 4] tensor; every head shares the one CSR (one forward launch)."""
        pat = torch.as_tensor(patterns, dtype=torch.int32).reshape(self.H, 4).contiguous().to(self.device)
        csr = self.new_csr()
        fpsa.pattern_mask(self.grid, self.tile, self.B, self.H, pat, csr.row_ptr, csr.col_idx,
                          self.workspace(), stream=stream)
        return csr

    def retained_mass(self, mass, csr: Csr, out=None, stream=None):
        """Share of each row's block mass [B, H, nb, nb] held by the CSR's blocks
        (the frozen indices' coverage at a later step): float32 [B, H, nb]."""
        out = torch.empty((self.B, self.H, self.nb), dtype=torch.float32, device=self.device) if out is None else out
        fpsa.retained_mass(mass, self.R, self.nb, csr.row_ptr, csr.col_idx, out, stream=stream)
        return out

    # ------------------------------------------------------------------ attention
    def forward(self, qt, kt, vt, csr: Csr, q_scale=None, k_scale=None, out=None, lse=None, out_f32=None,
                stream=None):
        """Tiled bf16 output; optionally lse and a float32 copy of the output (both
        for the backward)."""
        out = torch.empty(self.tiled_shape(), dtype=torch.bfloat16, device=self.device) if out is None else out
        fpsa.sparse_attn_fwd(qt, kt, vt, csr.row_ptr, csr.col_idx, self.grid, self.tile, self.B, self.H,
                             self.D, self.scale, out, q_scale=q_scale, k_scale=k_scale, lse=lse, o_f32=out_f32,
                             stream=stream)
        return out

    # ------------------------------------------------------------------ backward
    def transpose(self, csr: Csr, stream=None) -> Csr:
        """Column view of a CSR (per key block, the query blocks keeping it), the
        index lists the key-gradient pass walks."""
        csc = self.new_csr()
        ws = torch.empty(max(fpsa.transpose_workspace_bytes(self.R, self.nb), 1), dtype=torch.uint8,
                         device=self.device)
        fpsa.csr_transpose(csr.row_ptr, csr.col_idx, self.B, self.H, self.nb, csc.row_ptr, csc.col_idx, ws,
                           stream=stream)
        return csc

    def backward(self, qt, kt, vqk, ot, gt, lse, csr: Csr, csc: Csr, grads=None, workspace=None, stream=None,
                 q_scale=None, k_scale=None):
        """Gradients (dq, dk, dv) in tiled rows bf16 from Q, K, V and dO in the QK
        layout, the forward's tiled output (bf16, or its float32 copy for a more
        accurate delta) and lse, the CSR and its transpose."""
        if grads is None:
            grads = tuple(torch.empty(self.tiled_shape(), dtype=torch.bfloat16, device=self.device)
                          for _ in range(3))
        ws = workspace
        if ws is None:
            ws = torch.empty(fpsa.bwd_workspace_bytes(self.B, self.H, self.grid, self.tile), dtype=torch.uint8,
                             device=self.device)
        fpsa.sparse_attn_bwd(qt, kt, vqk, ot, gt, lse, csr.row_ptr, csr.col_idx, csc.row_ptr, csc.col_idx,
                             self.grid, self.tile, self.B, self.H, self.D, self.scale, *grads, ws, stream=stream,
                             q_scale=q_scale, k_scale=k_scale)
        return grads

    def run(self, q, k, v, thr_num=99, thr_den=100, out_dtype=torch.bfloat16):
        """Full path on raster Q, K, V: returns (raster O, CSR, masses)."""
        qt, kt, vt = self.tile_qk(q), self.tile_qk(k), self.tile_vt(v)
        mass = self.block_mass(qt, kt)
        csr = self.select(mass, thr_num, thr_den)
        ot = self.forward(qt, kt, vt, csr)
        return self.untile(ot, out_dtype), csr, mass


@dataclass
class Clusters:
    """One k-means clustering of the tokens of every (b, h) slice and its block layout."""
    assign: torch.Tensor        # int32 [B, H, N]
    centroids: torch.Tensor     # float64 [B, H, C, D]
    counts: torch.Tensor        # int32 [B, H, C]
    member_off: torch.Tensor    # int32 [B*H*C + 1]
    members: torch.Tensor       # int32 [B*H*N]
    slot_token: torch.Tensor    # int32 [B, H, NB*64]
    blk_off: torch.Tensor       # int32 [B, H, C+1]
    blk_count: torch.Tensor     # int32 [B, H, NB]


class SemanticSparseAttention:
    """Attention after a semantic-aware permutation [Sparse VideoGen2: Accelerate
    Video Generation with Sparse Attention via Semantic-Aware Permutation, Abstract]:
    per (b, h), k-means over the query vectors (Cq clusters) and over the key vectors
    (Ck clusters), each cluster laid out in whole 64-token blocks, cluster masses
    estimated from centroids and sizes, the top-p key clusters kept per query cluster
    (the same exact cut as the block selection), and the block-sparse forward over the
    resulting blocks. Everything is recomputed per call (the clustering follows the
    inputs)."""

    def __init__(self, N, B, H, D, Cq, Ck, iters=8, thr_num=9, thr_den=10, device="cuda", softmax_scale=None):
        self.N, self.B, self.H, self.D = int(N), int(B), int(H), int(D)
        self.Cq, self.Ck, self.iters = int(Cq), int(Ck), int(iters)
        self.thr = (int(thr_num), int(thr_den))
        self.device = torch.device(device)
        self.scale = float(softmax_scale) if softmax_scale is not None else 1.0 / math.sqrt(self.D)
        self.NB = -(-self.N // 64) + max(self.Cq, self.Ck)   # any clustering fits

    def tiled_shape(self):
        return (self.B, self.H, self.NB * 64, self.D)

    def cluster(self, x, C, stream=None) -> Clusters:
        B, H, N, D, NB, dev = self.B, self.H, self.N, self.D, self.NB, self.device
        i32 = dict(dtype=torch.int32, device=dev)
        c = Clusters(torch.empty((B, H, N), **i32), torch.empty((B, H, C, D), dtype=torch.float64, device=dev),
                     torch.empty((B, H, C), **i32), torch.empty(B * H * C + 1, **i32), torch.empty(B * H * N, **i32),
                     torch.empty((B, H, NB * 64), **i32), torch.empty((B, H, C + 1), **i32),
                     torch.empty((B, H, NB), **i32))
        ws = torch.empty(max(fpsa.kmeans_workspace_bytes(B, H, N, C), 1), dtype=torch.uint8, device=dev)
        fpsa.kmeans(x, B, N, H, D, C, self.iters, c.assign, c.centroids, c.counts, c.member_off, c.members, ws,
                    stream=stream)
        fpsa.cluster_layout(c.member_off, c.members, B, H, N, C, NB, c.slot_token, c.blk_off, c.blk_count,
                            stream=stream)
        return c

    def gather(self, x, clusters: Clusters, layout, stream=None):
        out = torch.empty(self.tiled_shape(), dtype=torch.bfloat16, device=self.device)
        fpsa.gather_tiles(x, clusters.slot_token, self.B, self.N, self.H, self.D, self.NB, layout, out, stream=stream)
        return out

    def cluster_mass(self, qc: Clusters, kc: Clusters, stream=None):
        est = torch.empty((self.B, self.H, self.Cq, self.Ck), dtype=torch.float32, device=self.device)
        fpsa.cluster_mass(qc.centroids, qc.counts, kc.centroids, kc.counts, self.B, self.H, self.Cq, self.Ck,
                          self.D, self.scale, est, stream=stream)
        return est

    def select_clusters(self, est, stream=None) -> Csr:
        R = self.B * self.H * self.Cq
        csr = Csr(torch.empty(R + 1, dtype=torch.int32, device=self.device),
                  torch.empty(R * self.Ck, dtype=torch.int32, device=self.device))
        ws = torch.empty(max(fpsa.select_workspace_bytes(R, self.Ck), 1), dtype=torch.uint8, device=self.device)
        fpsa.select_blocks(est, R, self.Ck, self.thr[0], self.thr[1], csr.row_ptr, csr.col_idx, ws, stream=stream)
        return csr

    def block_csr(self, ccsr: Csr, qc: Clusters, kc: Clusters, stream=None) -> Csr:
        R = self.B * self.H * self.NB
        csr = Csr(torch.empty(R + 1, dtype=torch.int32, device=self.device),
                  torch.empty(R * self.NB, dtype=torch.int32, device=self.device))
        ws = torch.empty(R, dtype=torch.int32, device=self.device)
        fpsa.cluster_blocks(ccsr.row_ptr, ccsr.col_idx, qc.blk_off, kc.blk_off, self.B, self.H, self.Cq, self.Ck,
                            self.NB, csr.row_ptr, csr.col_idx, ws, stream=stream)
        return csr

    def forward(self, qt, kt, vt, kc: Clusters, csr: Csr, out=None, lse=None, stream=None):
        out = torch.empty(self.tiled_shape(), dtype=torch.bfloat16, device=self.device) if out is None else out
        fpsa.sparse_attn_fwd_varlen(qt, kt, vt, kc.blk_count, csr.row_ptr, csr.col_idx, self.B, self.H, self.D,
                                    self.NB, self.scale, out, lse=lse, stream=stream)
        return out

    def scatter(self, ot, qc: Clusters, dtype=torch.bfloat16, stream=None):
        out = torch.empty((self.B, self.N, self.H, self.D), dtype=dtype, device=self.device)
        fpsa.scatter_tiles(ot, qc.slot_token, self.B, self.N, self.H, self.D, self.NB, out, stream=stream)
        return out

    def run(self, q, k, v, out_dtype=torch.bfloat16, stream=None):
        """Raster Q, K, V [B, N, H, D] -> (raster O, dict of the intermediate results)."""
        qc, kc = self.cluster(q, self.Cq, stream), self.cluster(k, self.Ck, stream)
        qt = self.gather(q, qc, fpsa.LAYOUT_QK, stream)
        kt = self.gather(k, kc, fpsa.LAYOUT_QK, stream)
        vt = self.gather(v, kc, fpsa.LAYOUT_VT, stream)
        est = self.cluster_mass(qc, kc, stream)
        ccsr = self.select_clusters(est, stream)
        csr = self.block_csr(ccsr, qc, kc, stream)
        ot = self.forward(qt, kt, vt, kc, csr, stream=stream)
        return self.scatter(ot, qc, out_dtype, stream), dict(qc=qc, kc=kc, est=est, ccsr=ccsr, csr=csr, ot=ot)
