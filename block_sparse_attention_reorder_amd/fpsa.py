"""Thin ctypes binding of libfpsa.so (include/fpsa.h): argument marshalling only.

Each function takes torch tensors that already live on the GPU (PyTorch provides
device memory and streams), checks dtype/shape/contiguity, and passes raw device
pointers plus the current HIP stream to the C ABI. Every computation runs in the
library's HIP kernels; there is no fallback. A non-OK status raises FpsaError.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# FPSA_LIB names another build of the same library (the host-sanitized one)
LIB_PATH = os.environ.get("FPSA_LIB") or os.path.join(HERE, "libfpsa.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_HIP = 0, 1, 2, 3, 4
F32, BF16, FP8_E4M3 = 0, 1, 2
LAYOUT_ROWS, LAYOUT_VT, LAYOUT_QK = 0, 1, 2
MAX_SELECT_BLOCKS = 4096

EXPORTED = [
    "fpsa_num_blocks", "fpsa_status_string", "fpsa_version", "fpsa_select_workspace_bytes",
    "fpsa_mass_workspace_bytes",
    "fpsa_tile_reorder", "fpsa_block_mass", "fpsa_select_blocks", "fpsa_structured_mask",
    "fpsa_pattern_mask", "fpsa_retained_mass", "fpsa_sparse_attn_fwd",
    "fpsa_csr_transpose", "fpsa_transpose_workspace_bytes", "fpsa_sparse_attn_bwd",
    "fpsa_bwd_workspace_bytes", "fpsa_kmeans", "fpsa_kmeans_workspace_bytes", "fpsa_cluster_layout",
    "fpsa_gather_tiles",
    "fpsa_scatter_tiles", "fpsa_cluster_mass", "fpsa_cluster_blocks", "fpsa_sparse_attn_fwd_varlen",
    "fpsa_dequantize_tiles", "fpsa_select_blocks_noalloc",
]
SELECT_NOALLOC_MAX_ROWS = 1 << 20


class FpsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class Grid(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32),
                ("tile_t", ctypes.c_int32), ("tile_h", ctypes.c_int32), ("tile_w", ctypes.c_int32)]

    @classmethod
    def of(cls, grid, tile) -> "Grid":
        return cls(*[int(x) for x in grid], *[int(x) for x in tile])


_lib = None


def lib() -> ctypes.CDLL:
    """Load the built library; raise if it was never built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_reorder_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float
        gp = ctypes.POINTER(Grid)
        L.fpsa_num_blocks.restype = i32
        L.fpsa_num_blocks.argtypes = [gp]
        L.fpsa_status_string.restype = ctypes.c_char_p
        L.fpsa_status_string.argtypes = [i32]
        L.fpsa_version.restype = i32
        L.fpsa_version.argtypes = []
        L.fpsa_select_workspace_bytes.restype = ctypes.c_size_t
        L.fpsa_select_workspace_bytes.argtypes = [i64, i32]
        L.fpsa_tile_reorder.restype = i32
        L.fpsa_tile_reorder.argtypes = [vp, i32, vp, i32, i32, vp, i32, i32, i32, gp, i32, vp]
        L.fpsa_dequantize_tiles.restype = i32
        L.fpsa_dequantize_tiles.argtypes = [vp, vp, i32, i32, i32, gp, vp, vp]
        L.fpsa_block_mass.restype = i32
        L.fpsa_block_mass.argtypes = [vp, vp, i32, i32, i32, gp, f32, vp, vp, vp, ctypes.c_size_t, vp]
        L.fpsa_mass_workspace_bytes.restype = ctypes.c_size_t
        L.fpsa_mass_workspace_bytes.argtypes = [i32, i32, gp]
        L.fpsa_select_blocks.restype = i32
        L.fpsa_select_blocks.argtypes = [vp, i64, i32, u32, u32, vp, vp, i64, vp, ctypes.c_size_t, vp]
        L.fpsa_select_blocks_noalloc.restype = i32
        L.fpsa_select_blocks_noalloc.argtypes = [vp, i64, i32, u32, u32, vp, vp, i64, vp]
        L.fpsa_structured_mask.restype = i32
        L.fpsa_structured_mask.argtypes = [gp, i32, vp, vp, i64, vp, ctypes.c_size_t, vp]
        L.fpsa_sparse_attn_fwd.restype = i32
        L.fpsa_pattern_mask.restype = i32
        L.fpsa_pattern_mask.argtypes = [gp, i32, i32, vp, vp, vp, i64, vp, ctypes.c_size_t, vp]
        L.fpsa_retained_mass.restype = i32
        L.fpsa_retained_mass.argtypes = [vp, i64, i32, vp, vp, vp, vp]
        L.fpsa_csr_transpose.restype = i32
        L.fpsa_csr_transpose.argtypes = [vp, vp, i32, i32, i32, vp, vp, i64, vp, ctypes.c_size_t, vp]
        L.fpsa_transpose_workspace_bytes.restype = ctypes.c_size_t
        L.fpsa_transpose_workspace_bytes.argtypes = [i64, i32]
        L.fpsa_sparse_attn_bwd.restype = i32
        L.fpsa_sparse_attn_bwd.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, gp, f32,
                                           vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.fpsa_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.fpsa_bwd_workspace_bytes.argtypes = [i32, i32, gp]
        L.fpsa_kmeans.restype = i32
        L.fpsa_kmeans.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.fpsa_kmeans_workspace_bytes.restype = ctypes.c_size_t
        L.fpsa_kmeans_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.fpsa_cluster_layout.restype = i32
        L.fpsa_cluster_layout.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
        L.fpsa_gather_tiles.restype = i32
        L.fpsa_gather_tiles.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, i32, vp, vp]
        L.fpsa_scatter_tiles.restype = i32
        L.fpsa_scatter_tiles.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, i32, vp]
        L.fpsa_cluster_mass.restype = i32
        L.fpsa_cluster_mass.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp]
        L.fpsa_cluster_blocks.restype = i32
        L.fpsa_cluster_blocks.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, i64, vp,
                                          ctypes.c_size_t, vp]
        L.fpsa_sparse_attn_fwd_varlen.restype = i32
        L.fpsa_sparse_attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, vp, vp, vp]
        L.fpsa_sparse_attn_fwd.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, gp, f32,
                                           vp, vp, vp, vp]
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().fpsa_status_string(int(s)).decode()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise FpsaError(status, what)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.uint8: FP8_E4M3, torch.float8_e4m3fn: FP8_E4M3}


# --------------------------------------------------------------------------- host-only

def num_blocks(grid, tile) -> int:
    g = Grid.of(grid, tile)
    return int(lib().fpsa_num_blocks(ctypes.byref(g)))


def select_workspace_bytes(R: int, nb: int) -> int:
    return int(lib().fpsa_select_workspace_bytes(int(R), int(nb)))


def mass_workspace_bytes(B: int, H: int, grid, tile) -> int:
    g = Grid.of(grid, tile)
    return int(lib().fpsa_mass_workspace_bytes(int(B), int(H), ctypes.byref(g)))


def version() -> int:
    return int(lib().fpsa_version())


# --------------------------------------------------------------------------- device calls

def tile_reorder(src, dst, grid, tile, B, H, D, *, inverse=False, layout=LAYOUT_ROWS,
                 dst_scale=None, stream=None) -> None:
    """fpsa_tile_reorder; dtypes are taken from the tensors (uint8 = e4m3 bytes)."""
    g = Grid.of(grid, tile)
    s = lib().fpsa_tile_reorder(_ptr(src), _DT[src.dtype], _ptr(dst), _DT[dst.dtype], int(layout),
                                _ptr(dst_scale), int(B), int(H), int(D), ctypes.byref(g),
                                1 if inverse else 0, _stream(stream))
    _check(s, "fpsa_tile_reorder")


def dequantize_tiles(src, scale, grid, tile, B, H, D, dst, stream=None) -> None:
    """fpsa_dequantize_tiles: e4m3 QK tiles (uint8) and their scales -> bf16 QK tiles
    (scale None: the code values, the form the FP8 backward takes)."""
    if src.dtype not in (torch.uint8, torch.float8_e4m3fn) or (scale is not None and scale.dtype != torch.float32):
        raise ValueError("src e4m3 bytes, scale float32 or None (code values)")
    if dst.dtype != torch.bfloat16:
        raise ValueError("dst bf16")
    g = Grid.of(grid, tile)
    s = lib().fpsa_dequantize_tiles(_ptr(src), _ptr(scale), int(B), int(H), int(D), ctypes.byref(g),
                                    _ptr(dst), _stream(stream))
    _check(s, "fpsa_dequantize_tiles")


def block_mass(q_tiled, k_tiled, grid, tile, B, H, D, softmax_scale, mass, workspace, lse=None,
               stream=None) -> None:
    if q_tiled.dtype != torch.bfloat16 or k_tiled.dtype != torch.bfloat16:
        raise ValueError("block_mass takes bf16 tiled Q and K")
    if mass.dtype != torch.float32 or (lse is not None and lse.dtype != torch.float32):
        raise ValueError("mass and lse are float32")
    g = Grid.of(grid, tile)
    s = lib().fpsa_block_mass(_ptr(q_tiled), _ptr(k_tiled), int(B), int(H), int(D), ctypes.byref(g),
                              float(softmax_scale), _ptr(mass), _ptr(lse), _ptr(workspace),
                              int(workspace.numel() * workspace.element_size()), _stream(stream))
    _check(s, "fpsa_block_mass")


def select_blocks(mass, R, nb, thr_num, thr_den, row_ptr, col_idx, workspace, stream=None) -> None:
    if mass.dtype != torch.float32 or row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("mass float32, row_ptr/col_idx int32")
    s = lib().fpsa_select_blocks(_ptr(mass), int(R), int(nb), int(thr_num), int(thr_den), _ptr(row_ptr),
                                 _ptr(col_idx), int(col_idx.numel()), _ptr(workspace),
                                 int(workspace.numel() * workspace.element_size()), _stream(stream))
    _check(s, "fpsa_select_blocks")


def select_blocks_noalloc(mass, R, nb, thr_num, thr_den, row_ptr, col_idx, stream=None) -> None:
    """fpsa_select_blocks on the library's static device scratch (no workspace)."""
    if mass.dtype != torch.float32 or row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("mass float32, row_ptr/col_idx int32")
    s = lib().fpsa_select_blocks_noalloc(_ptr(mass), int(R), int(nb), int(thr_num), int(thr_den), _ptr(row_ptr),
                                         _ptr(col_idx), int(col_idx.numel()), _stream(stream))
    _check(s, "fpsa_select_blocks_noalloc")


def structured_mask(grid, tile, copies, row_ptr, col_idx, workspace, stream=None) -> None:
    g = Grid.of(grid, tile)
    s = lib().fpsa_structured_mask(ctypes.byref(g), int(copies), _ptr(row_ptr), _ptr(col_idx),
                                   int(col_idx.numel()), _ptr(workspace),
                                   int(workspace.numel() * workspace.element_size()), _stream(stream))
    _check(s, "fpsa_structured_mask")


def pattern_mask(grid, tile, B, H, patterns, row_ptr, col_idx, workspace, stream=None) -> None:
    """patterns: int32 device tensor [H, 4] = (band, period, stripe, dense) per head."""
    if patterns.dtype != torch.int32 or tuple(patterns.shape) != (int(H), 4) or not patterns.is_contiguous():
        raise ValueError("patterns must be a contiguous int32 [H, 4] tensor")
    g = Grid.of(grid, tile)
    s = lib().fpsa_pattern_mask(ctypes.byref(g), int(B), int(H), _ptr(patterns), _ptr(row_ptr),
                                _ptr(col_idx), int(col_idx.numel()), _ptr(workspace),
                                int(workspace.numel() * workspace.element_size()), _stream(stream))
    _check(s, "fpsa_pattern_mask")


def retained_mass(mass, R, nb, row_ptr, col_idx, out, stream=None) -> None:
    if mass.dtype != torch.float32 or out.dtype != torch.float32:
        raise ValueError("mass and out float32")
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr/col_idx int32")
    if mass.numel() < int(R) * int(nb) or out.numel() < int(R) or row_ptr.numel() < int(R) + 1:
        raise ValueError("mass [R, nb], out [R] and row_ptr [R + 1] are too small")
    s = lib().fpsa_retained_mass(_ptr(mass), int(R), int(nb), _ptr(row_ptr), _ptr(col_idx), _ptr(out),
                                 _stream(stream))
    _check(s, "fpsa_retained_mass")


def transpose_workspace_bytes(R: int, nb: int) -> int:
    return int(lib().fpsa_transpose_workspace_bytes(int(R), int(nb)))


def bwd_workspace_bytes(B: int, H: int, grid, tile) -> int:
    g = Grid.of(grid, tile)
    return int(lib().fpsa_bwd_workspace_bytes(int(B), int(H), ctypes.byref(g)))


def csr_transpose(row_ptr, col_idx, B, H, nb, col_ptr, row_idx, workspace, stream=None) -> None:
    for t in (row_ptr, col_idx, col_ptr, row_idx):
        if t.dtype != torch.int32:
            raise ValueError("CSR arrays are int32")
    s = lib().fpsa_csr_transpose(_ptr(row_ptr), _ptr(col_idx), int(B), int(H), int(nb), _ptr(col_ptr),
                                 _ptr(row_idx), int(row_idx.numel()), _ptr(workspace),
                                 int(workspace.numel() * workspace.element_size()), _stream(stream))
    _check(s, "fpsa_csr_transpose")


def sparse_attn_bwd(q, k, v, o, dout, lse, row_ptr, col_idx, col_ptr, row_idx, grid, tile, B, H, D,
                    softmax_scale, dq, dk, dv, workspace, stream=None, q_scale=None, k_scale=None) -> None:
    for t in (q, k, v, dout, dq, dk, dv):
        if t.dtype != torch.bfloat16:
            raise ValueError("q, k, v, dout and the gradients are bf16")
    if o.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("o is bf16 or float32")
    if lse.dtype != torch.float32:
        raise ValueError("lse float32")
    g = Grid.of(grid, tile)
    for t in (q_scale, k_scale):
        if t is not None and t.dtype != torch.float32:
            raise ValueError("tile scales float32")
    s = lib().fpsa_sparse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _DT[o.dtype], _ptr(dout), _ptr(lse), _ptr(row_ptr),
                                   _ptr(col_idx), _ptr(col_ptr), _ptr(row_idx), _ptr(q_scale), _ptr(k_scale),
                                   int(B), int(H), int(D),
                                   ctypes.byref(g), float(softmax_scale), _ptr(dq), _ptr(dk), _ptr(dv),
                                   _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                   _stream(stream))
    _check(s, "fpsa_sparse_attn_bwd")


def sparse_attn_fwd(q, k, v, row_ptr, col_idx, grid, tile, B, H, D, softmax_scale, o, *,
                    q_scale=None, k_scale=None, lse=None, o_f32=None, stream=None) -> None:
    qk_dt = _DT[q.dtype]
    if _DT[k.dtype] != qk_dt or v.dtype != torch.bfloat16 or o.dtype != torch.bfloat16:
        raise ValueError("q/k same dtype (bf16 or e4m3 bytes), v and o bf16")
    if o_f32 is not None and o_f32.dtype != torch.float32:
        raise ValueError("o_f32 float32")
    g = Grid.of(grid, tile)
    s = lib().fpsa_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), qk_dt, _ptr(q_scale), _ptr(k_scale),
                                   _ptr(row_ptr), _ptr(col_idx), int(B), int(H), int(D), ctypes.byref(g),
                                   float(softmax_scale), _ptr(o), _ptr(lse), _ptr(o_f32), _stream(stream))
    _check(s, "fpsa_sparse_attn_fwd")


# --------------------------------------------------------------------------- k-means permutation

def _i32(*ts):
    for t in ts:
        if t.dtype != torch.int32:
            raise ValueError("index arrays are int32")


def kmeans_workspace_bytes(B, H, N, C) -> int:
    return int(lib().fpsa_kmeans_workspace_bytes(int(B), int(H), int(N), int(C)))


def kmeans(x, B, N, H, D, C, iters, assign, centroids, counts, member_off, members, workspace,
           stream=None) -> None:
    _i32(assign, counts, member_off, members)
    if centroids.dtype != torch.float64:
        raise ValueError("centroids float64")
    s = lib().fpsa_kmeans(_ptr(x), _DT[x.dtype], int(B), int(N), int(H), int(D), int(C), int(iters),
                          _ptr(assign), _ptr(centroids), _ptr(counts), _ptr(member_off), _ptr(members),
                          _ptr(workspace), int(workspace.numel() * workspace.element_size()), _stream(stream))
    _check(s, "fpsa_kmeans")


def cluster_layout(member_off, members, B, H, N, C, NB, slot_token, blk_off, blk_count, stream=None) -> None:
    _i32(member_off, members, slot_token, blk_off, blk_count)
    s = lib().fpsa_cluster_layout(_ptr(member_off), _ptr(members), int(B), int(H), int(N), int(C), int(NB),
                                  _ptr(slot_token), _ptr(blk_off), _ptr(blk_count), _stream(stream))
    _check(s, "fpsa_cluster_layout")


def gather_tiles(src, slot_token, B, N, H, D, NB, layout, dst, stream=None) -> None:
    _i32(slot_token)
    if dst.dtype != torch.bfloat16:
        raise ValueError("gathered tiles are bf16")
    s = lib().fpsa_gather_tiles(_ptr(src), _DT[src.dtype], _ptr(slot_token), int(B), int(N), int(H), int(D),
                                int(NB), int(layout), _ptr(dst), _stream(stream))
    _check(s, "fpsa_gather_tiles")


def scatter_tiles(src, slot_token, B, N, H, D, NB, dst, stream=None) -> None:
    _i32(slot_token)
    if src.dtype != torch.bfloat16:
        raise ValueError("tiled rows are bf16")
    s = lib().fpsa_scatter_tiles(_ptr(src), _ptr(slot_token), int(B), int(N), int(H), int(D), int(NB),
                                 _ptr(dst), _DT[dst.dtype], _stream(stream))
    _check(s, "fpsa_scatter_tiles")


def cluster_mass(cq, nq, ck, nk, B, H, Cq, Ck, D, softmax_scale, est, stream=None) -> None:
    _i32(nq, nk)
    if cq.dtype != torch.float64 or ck.dtype != torch.float64 or est.dtype != torch.float32:
        raise ValueError("centroids float64, est float32")
    s = lib().fpsa_cluster_mass(_ptr(cq), _ptr(nq), _ptr(ck), _ptr(nk), int(B), int(H), int(Cq), int(Ck),
                                int(D), float(softmax_scale), _ptr(est), _stream(stream))
    _check(s, "fpsa_cluster_mass")


def cluster_blocks(crow_ptr, ccol_idx, qoff, koff, B, H, Cq, Ck, NB, row_ptr, col_idx, workspace,
                   stream=None) -> None:
    _i32(crow_ptr, ccol_idx, qoff, koff, row_ptr, col_idx)
    s = lib().fpsa_cluster_blocks(_ptr(crow_ptr), _ptr(ccol_idx), _ptr(qoff), _ptr(koff), int(B), int(H),
                                  int(Cq), int(Ck), int(NB), _ptr(row_ptr), _ptr(col_idx), int(col_idx.numel()),
                                  _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                  _stream(stream))
    _check(s, "fpsa_cluster_blocks")


def sparse_attn_fwd_varlen(q, k, v, key_counts, row_ptr, col_idx, B, H, D, NB, softmax_scale, o, *, lse=None,
                           o_f32=None, stream=None) -> None:
    _i32(key_counts, row_ptr, col_idx)
    for t in (q, k, v, o):
        if t.dtype != torch.bfloat16:
            raise ValueError("q, k, v and o are bf16")
    s = lib().fpsa_sparse_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(key_counts), _ptr(row_ptr),
                                          _ptr(col_idx), int(B), int(H), int(D), int(NB), float(softmax_scale),
                                          _ptr(o), _ptr(lse), _ptr(o_f32), _stream(stream))
    _check(s, "fpsa_sparse_attn_fwd_varlen")
