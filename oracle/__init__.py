"""CPU oracle: plain float64 definitions of what the block-sparse path computes.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, the smoke check and the benchmark's
CPU-baseline leg import this package; the product path never does. It shares no
code with the HIP library: geometry, masses, selection, masked attention, FP8
quantization, the structured mask, the retained-mass monitor, the fixed
diagonal / multi-diagonal / stripe patterns, the gradients of masked attention, the
block-CSR transpose, the k-means semantic permutation (clusters, layout, cluster
masses, cluster attention) and bf16 rounding are each written here from their definitions
(``fpsa_oracle.c``), over raster-ordered tokens.

Parity pins (tests/test_oracle_pins.py) tie each function to something other than
itself: closed forms, invariants, brute force on tiny inputs, textbook softmax
attention computed by a library routine, and the published e4m3 code table.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fpsa_oracle.c")
# FPSA_ORACLE_SANITIZE=1 selects a build with AddressSanitizer and UndefinedBehavior-
# Sanitizer (the process must preload gcc's libasan and libubsan); the arithmetic is
# the same source
_SANITIZE = os.environ.get("FPSA_ORACLE_SANITIZE", "") not in ("", "0")
_LIB_PATH = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")
_SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=undefined"]
_lock = threading.Lock()
_lib = None

_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_vp = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP over independent rows)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        opt = _SAN_FLAGS if _SANITIZE else ["-O2"]
        subprocess.check_call(["gcc", *opt, "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB_PATH)
            L.orc_num_blocks.restype = ctypes.c_int64
            L.orc_num_blocks.argtypes = [ctypes.c_int] * 6
            L.orc_token_blocks.restype = None
            L.orc_token_blocks.argtypes = [ctypes.c_int] * 6 + [_i32p, _vp]
            L.orc_dense_attention.restype = None
            L.orc_dense_attention.argtypes = [_f32p, _f32p, _f32p] + [ctypes.c_int] * 4 + [
                ctypes.c_double, _vp, ctypes.c_int, _f64p]
            L.orc_block_mass.restype = None
            L.orc_block_mass.argtypes = [_f32p, _f32p] + [ctypes.c_int] * 4 + [
                _i32p, ctypes.c_int, ctypes.c_double, _vp, ctypes.c_int, _f64p]
            L.orc_mass_key.restype = ctypes.c_uint64
            L.orc_mass_key.argtypes = [ctypes.c_float]
            L.orc_select_blocks.restype = ctypes.c_int64
            L.orc_select_blocks.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32,
                                            ctypes.c_uint32, _i32p, _i32p]
            L.orc_cut_margin.restype = None
            L.orc_cut_margin.argtypes = [_f64p, ctypes.c_int64, ctypes.c_int, ctypes.c_double, _f64p]
            L.orc_masked_attention.restype = None
            L.orc_masked_attention.argtypes = [_f32p, _f32p, _f32p] + [ctypes.c_int] * 4 + [
                _i32p, ctypes.c_int, ctypes.c_double, _i32p, _i32p, _vp, ctypes.c_int, _f64p, _i32p]
            L.orc_e4m3_decode.restype = ctypes.c_double
            L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
            L.orc_e4m3_encode.restype = ctypes.c_uint8
            L.orc_e4m3_encode.argtypes = [ctypes.c_double]
            L.orc_fp8_tile_quantize.restype = None
            L.orc_fp8_tile_quantize.argtypes = [_f32p] + [ctypes.c_int] * 4 + [_i32p, ctypes.c_int, _f32p, _f32p]
            L.orc_fp8_tile_codes.restype = None
            L.orc_fp8_tile_codes.argtypes = [_f32p] + [ctypes.c_int] * 4 + [_i32p, ctypes.c_int, _u8p, _f32p]
            L.orc_round_bf16.restype = None
            L.orc_round_bf16.argtypes = [_f32p, ctypes.c_int64, _f32p]
            L.orc_structured_mask.restype = ctypes.c_int64
            L.orc_structured_mask.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _i32p]
            L.orc_retained_mass.restype = None
            L.orc_retained_mass.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int, _i32p, _i32p, _f64p]
            L.orc_pattern_mask.restype = ctypes.c_int64
            L.orc_masked_attention_bwd.restype = None
            L.orc_masked_attention_bwd.argtypes = [_f32p] * 4 + [ctypes.c_int] * 4 + [
                _i32p, ctypes.c_int, ctypes.c_double, _i32p, _i32p, _f64p, _f64p, _f64p, _vp, _vp, _vp]
            L.orc_masked_attention_bwd_dq.restype = None
            L.orc_masked_attention_bwd_dq.argtypes = [_f32p] * 4 + [ctypes.c_int] * 4 + [
                _i32p, ctypes.c_int, ctypes.c_double, _i32p, _i32p, _i32p, ctypes.c_int, _f64p, _vp, _i32p]
            L.orc_csr_transpose.restype = ctypes.c_int64
            L.orc_kmeans.restype = None
            L.orc_kmeans.argtypes = [_f32p] + [ctypes.c_int] * 6 + [_i32p, _f64p, _i32p]
            L.orc_kmeans_assign.restype = None
            L.orc_kmeans_assign.argtypes = [_f32p] + [ctypes.c_int] * 5 + [_f64p, _i32p, _vp, _vp, _vp]
            L.orc_kmeans_means.restype = None
            L.orc_kmeans_means.argtypes = [_f32p] + [ctypes.c_int] * 5 + [_i32p, _f64p, _f64p, _i32p, _vp]
            L.orc_cluster_layout.restype = ctypes.c_int
            L.orc_cluster_layout.argtypes = [_i32p] + [ctypes.c_int] * 5 + [_i32p, _i32p, _i32p]
            L.orc_cluster_mass.restype = None
            L.orc_cluster_mass.argtypes = [_f64p, _i32p, _f64p, _i32p] + [ctypes.c_int] * 5 + [ctypes.c_double, _f64p]
            L.orc_cluster_blocks.restype = ctypes.c_int64
            L.orc_cluster_blocks.argtypes = [_i32p] * 4 + [ctypes.c_int] * 5 + [_i32p, _i32p]
            L.orc_cluster_attention.restype = None
            L.orc_cluster_attention.argtypes = [_f32p] * 3 + [ctypes.c_int] * 4 + [_i32p, _i32p, ctypes.c_int,
                                                                                    ctypes.c_int, ctypes.c_double,
                                                                                    _i32p, _i32p, _vp, ctypes.c_int,
                                                                                    _f64p]
            L.orc_csr_transpose.argtypes = [_i32p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _i32p]
            L.orc_pattern_mask.argtypes = [ctypes.c_int] * 3 + [_i32p, _i32p, _i32p]
            _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _opt_i32(a):
    """(pointer, count, keepalive) for an optional int32 index list."""
    if a is None:
        return None, 0, None
    arr = _c(a, np.int32)
    return arr.ctypes.data_as(ctypes.c_void_p), len(arr), arr


# --------------------------------------------------------------------------- geometry

def num_blocks(grid, tile) -> int:
    return int(lib().orc_num_blocks(*grid, *tile))


def token_blocks(grid, tile):
    """(block_of[N] int32, slot_of[N] int64) for the raster tokens of ``grid``."""
    T, Hg, Wg = grid
    N = T * Hg * Wg
    blk = np.empty(N, np.int32)
    slot = np.empty(N, np.int64)
    lib().orc_token_blocks(*grid, *tile, blk, slot.ctypes.data_as(ctypes.c_void_p))
    return blk, slot


def block_sizes(grid, tile):
    """Number of real tokens in every block."""
    blk, _ = token_blocks(grid, tile)
    return np.bincount(blk, minlength=num_blocks(grid, tile))


# --------------------------------------------------------------------------- attention

def dense_attention(q, k, v, scale, queries=None):
    """Full softmax attention; q, k, v raster [B, N, H, D]. Rows not in ``queries`` are 0."""
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    B, N, H, D = q.shape
    out = np.zeros((B, N, H, D), np.float64)
    p, n, keep = _opt_i32(queries)
    lib().orc_dense_attention(q, k, v, B, N, H, D, float(scale), p, n, out)
    return out


def block_mass(q, k, grid, tile, scale, qblocks=None):
    """Block masses [B, H, nsel, nb] float64 (rows for ``qblocks``, default all)."""
    q, k = _c(q, np.float32), _c(k, np.float32)
    B, N, H, D = q.shape
    blk, _ = token_blocks(grid, tile)
    nb = num_blocks(grid, tile)
    p, n, keep = _opt_i32(qblocks)
    count = n if qblocks is not None else nb
    out = np.empty((B, H, count, nb), np.float64)
    lib().orc_block_mass(q, k, B, N, H, D, blk, nb, float(scale), p, n, out)
    return out


def mass_key(m: float) -> int:
    return int(lib().orc_mass_key(float(m)))


def select_blocks(mass, thr_num=99, thr_den=100):
    """CSR (row_ptr[R+1], col_idx[nnz]) of the retained-mass selection of float32 rows."""
    m = _c(mass, np.float32)
    nb = m.shape[-1]
    m2 = m.reshape(-1, nb)
    R = m2.shape[0]
    row_ptr = np.zeros(R + 1, np.int32)
    col_idx = np.zeros(max(R * nb, 1), np.int32)
    nnz = lib().orc_select_blocks(m2, R, nb, thr_num, thr_den, row_ptr, col_idx)
    return row_ptr, col_idx[:nnz].copy()


def cut_margin(mass64, p=0.99):
    m = _c(mass64, np.float64)
    nb = m.shape[-1]
    m2 = m.reshape(-1, nb)
    out = np.empty(m2.shape[0], np.float64)
    lib().orc_cut_margin(m2, m2.shape[0], nb, float(p), out)
    return out


def masked_attention(q, k, v, grid, tile, scale, row_ptr, col_idx, qblocks=None):
    """Masked attention for the requested query blocks.

    Returns (out [B, H, nsel, 64, D] float64, token_of [B, H, nsel, 64] int32): row e
    of a block is its e-th real token in raster order (token_of = -1 past the end).
    """
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    B, N, H, D = q.shape
    blk, _ = token_blocks(grid, tile)
    nb = num_blocks(grid, tile)
    p, n, keep = _opt_i32(qblocks)
    count = n if qblocks is not None else nb
    out = np.empty((B, H, count, 64, D), np.float64)
    tok = np.empty((B, H, count, 64), np.int32)
    rp = _c(row_ptr, np.int32)
    ci = _c(col_idx, np.int32)
    if ci.size == 0:
        ci = np.zeros(1, np.int32)
    lib().orc_masked_attention(q, k, v, B, N, H, D, blk, nb, float(scale), rp, ci, p, n, out, tok)
    return out, tok


# --------------------------------------------------------------------------- fp8

def e4m3_decode(code: int) -> float:
    return float(lib().orc_e4m3_decode(int(code) & 0xFF))


def e4m3_encode(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(x)))


def fp8_tile_quantize(x, grid, tile):
    """(xhat [B, N, H, D] float32, scales [B, H, nb] float32) of per-tile e4m3 quantization."""
    x = _c(x, np.float32)
    B, N, H, D = x.shape
    blk, _ = token_blocks(grid, tile)
    nb = num_blocks(grid, tile)
    xhat = np.empty_like(x)
    scales = np.empty((B, H, nb), np.float32)
    lib().orc_fp8_tile_quantize(x, B, N, H, D, blk, nb, xhat, scales)
    return xhat, scales


def fp8_tile_codes(x, grid, tile):
    """(codes [B, N, H, D] uint8 raster, scales [B, H, nb] float32) of per-tile e4m3 quantization."""
    x = _c(x, np.float32)
    B, N, H, D = x.shape
    blk, _ = token_blocks(grid, tile)
    nb = num_blocks(grid, tile)
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty((B, H, nb), np.float32)
    lib().orc_fp8_tile_codes(x, B, N, H, D, blk, nb, codes, scales)
    return codes, scales


def round_bf16(x):
    """float32 array -> float32 array of its bf16 values (round to nearest even)."""
    x = _c(x, np.float32)
    out = np.empty_like(x)
    lib().orc_round_bf16(x.reshape(-1), x.size, out.reshape(-1))
    return out


def fp8_dequantized_bf16(x, grid, tile):
    """The dequantized e4m3 tile values (code value times tile scale, as float32)
    rounded to bf16: the Q and K the backward of the FP8 forward reads."""
    xhat, _ = fp8_tile_quantize(x, grid, tile)
    return round_bf16(xhat)


# --------------------------------------------------------------------------- structured mask

def structured_mask(gh, gw, copies=1):
    nb = gh * gw
    row_ptr = np.zeros(copies * nb + 1, np.int32)
    # each row keeps at most 3x3 + one row + one column of groups
    cap = copies * nb * (gw + gh + 9)
    col_idx = np.zeros(cap, np.int32)
    nnz = lib().orc_structured_mask(gh, gw, copies, row_ptr, col_idx)
    return row_ptr, col_idx[:nnz].copy()


# --------------------------------------------------------------------------- monitor and patterns

def retained_mass(mass, row_ptr, col_idx):
    """Per row: the sum of the row's block masses (rows x nb, any leading shape)
    over the distinct in-range indices its CSR row lists, in float64."""
    m = _c(mass, np.float32)
    nb = m.shape[-1]
    m = m.reshape(-1, nb)
    ci = _c(col_idx, np.int32) if len(col_idx) else np.zeros(1, np.int32)
    out = np.zeros(m.shape[0], np.float64)
    lib().orc_retained_mass(m, m.shape[0], nb, _c(row_ptr, np.int32), ci, out)
    return out


def pattern_mask(nb, B, H, patterns):
    """CSR of the per-head fixed patterns; patterns: H tuples (band, period, stripe, dense)."""
    pat = np.ascontiguousarray(np.asarray(patterns, np.int32).reshape(H, 4))
    row_ptr = np.zeros(B * H * nb + 1, np.int32)
    col_idx = np.zeros(max(B * H * nb * nb, 1), np.int32)
    nnz = lib().orc_pattern_mask(nb, B, H, pat, row_ptr, col_idx)
    return row_ptr, col_idx[:nnz].copy()


# --------------------------------------------------------------------------- backward

def masked_attention_bwd(q, k, v, dout, grid, tile, scale, row_ptr, col_idx, magnitudes=False):
    """(dq, dk, dv), raster [B, N, H, D] float64: gradients of masked attention for
    the upstream gradient dout; with magnitudes=True also (mq, mk, mv), the sums of
    the absolute values of the terms of each gradient element."""
    q, k, v, g = (_c(x, np.float32) for x in (q, k, v, dout))
    B, N, H, D = q.shape
    blk, _ = token_blocks(grid, tile)
    nb = num_blocks(grid, tile)
    n = 6 if magnitudes else 3
    arrs = [np.empty((B, N, H, D), np.float64) for _ in range(n)]
    ptrs = [a.ctypes.data for a in arrs[3:]] if magnitudes else [None, None, None]
    ci = _c(col_idx, np.int32) if len(col_idx) else np.zeros(1, np.int32)
    lib().orc_masked_attention_bwd(q, k, v, g, B, N, H, D, blk, nb, float(scale),
                                   _c(row_ptr, np.int32), ci, arrs[0], arrs[1], arrs[2], *ptrs)
    return tuple(arrs)


def masked_attention_bwd_dq(q, k, v, dout, grid, tile, scale, row_ptr, col_idx, qblocks,
                            magnitudes=False):
    """(dq [B, H, nsel, 64, D] float64, token_of [B, H, nsel, 64]) for the listed
    query blocks, rows ordered as in masked_attention; with magnitudes=True,
    (dq, mq, token_of)."""
    q, k, v, g = (_c(x, np.float32) for x in (q, k, v, dout))
    B, N, H, D = q.shape
    blk, _ = token_blocks(grid, tile)
    nb = num_blocks(grid, tile)
    qb = _c(qblocks, np.int32)
    dq = np.empty((B, H, len(qb), 64, D), np.float64)
    mq = np.empty_like(dq) if magnitudes else None
    tok = np.empty((B, H, len(qb), 64), np.int32)
    ci = _c(col_idx, np.int32) if len(col_idx) else np.zeros(1, np.int32)
    lib().orc_masked_attention_bwd_dq(q, k, v, g, B, N, H, D, blk, nb, float(scale),
                                      _c(row_ptr, np.int32), ci, qb, len(qb), dq,
                                      mq.ctypes.data if magnitudes else None, tok)
    return (dq, mq, tok) if magnitudes else (dq, tok)


def csr_transpose(row_ptr, col_idx, B, H, nb):
    """(col_ptr [B*H*nb + 1], row_idx [nnz]): per (b, h) the query blocks keeping each key block."""
    R = B * H * nb
    col_ptr = np.zeros(R + 1, np.int32)
    row_idx = np.zeros(max(len(col_idx), 1), np.int32)
    ci = _c(col_idx, np.int32) if len(col_idx) else np.zeros(1, np.int32)
    nnz = lib().orc_csr_transpose(_c(row_ptr, np.int32), ci, B, H, nb, col_ptr, row_idx)
    return col_ptr, row_idx[:nnz].copy()


# --------------------------------------------------------------------------- k-means permutation

def kmeans(x, C, iters):
    """(assign [B, H, N] int32, centroids [B, H, C, D] float64, counts [B, H, C]) of
    Lloyd's k-means per (b, h) over x [B, N, H, D]."""
    x = _c(x, np.float32)
    B, N, H, D = x.shape
    assign = np.zeros((B, H, N), np.int32)
    cent = np.zeros((B, H, C, D), np.float64)
    count = np.zeros((B, H, C), np.int32)
    lib().orc_kmeans(x, B, N, H, D, int(C), int(iters), assign, cent, count)
    return assign, cent, count


def kmeans_start(x, C):
    """Starting centroids [B, H, C, D] float64: centroid c is token floor(c N / C)."""
    x = _c(x, np.float32)
    B, N, H, D = x.shape
    idx = (np.arange(C, dtype=np.int64) * N) // C
    return np.ascontiguousarray(np.transpose(x[:, idx, :, :], (0, 2, 1, 3)).astype(np.float64))


def kmeans_assign(x, cent, other=None):
    """Nearest centroid of every token (least squared distance, ties to the lower
    cluster): assign [B, H, N]. With ``other`` (an assignment [B, H, N] to check),
    also (excess, tol) [B, H, N]: how much farther other's centroid is than the
    nearest, and the bound on evaluation error for the two distances; ``other`` is a
    valid choice where excess <= tol."""
    x = _c(x, np.float32)
    cent = _c(cent, np.float64)
    B, N, H, D = x.shape
    C = cent.shape[2]
    assign = np.zeros((B, H, N), np.int32)
    if other is None:
        lib().orc_kmeans_assign(x, B, N, H, D, C, cent, assign, None, None, None)
        return assign
    oth = _c(other, np.int32)
    excess = np.zeros((B, H, N), np.float64)
    tol = np.zeros((B, H, N), np.float64)
    lib().orc_kmeans_assign(x, B, N, H, D, C, cent, assign, oth.ctypes.data, excess.ctypes.data,
                            tol.ctypes.data)
    return assign, excess, tol


def kmeans_means(x, assign, cent_in):
    """(cent [B, H, C, D] float64, count [B, H, C], abs_sum [B, H, C, D]): members'
    means in token order (empty clusters keep cent_in) and the sums of |x| over the
    members."""
    x = _c(x, np.float32)
    cent_in = _c(cent_in, np.float64)
    B, N, H, D = x.shape
    C = cent_in.shape[2]
    cent = np.zeros_like(cent_in)
    count = np.zeros((B, H, C), np.int32)
    abs_sum = np.zeros_like(cent_in)
    lib().orc_kmeans_means(x, B, N, H, D, C, _c(assign, np.int32), cent_in, cent, count, abs_sum.ctypes.data)
    return cent, count, abs_sum


def blocks_for(N, C):
    """Blocks per head that any clustering of N tokens into C clusters fits in."""
    return -(-N // 64) + C


def cluster_layout(assign, C, NB):
    """(slot_token [B, H, NB*64], off [B, H, C+1], blk_count [B, H, NB])."""
    a = _c(assign, np.int32)
    B, H, N = a.shape
    st = np.zeros((B, H, NB * 64), np.int32)
    off = np.zeros((B, H, C + 1), np.int32)
    bc = np.zeros((B, H, NB), np.int32)
    if lib().orc_cluster_layout(a, B, H, N, int(C), int(NB), st, off, bc) != 0:
        raise ValueError("clusters need more than NB blocks")
    return st, off, bc


def cluster_mass(cq, nq, ck, nk, scale):
    """est [B, H, Cq, Ck] float64 from centroids and cluster sizes."""
    cq, ck = _c(cq, np.float64), _c(ck, np.float64)
    B, H, Cq, D = cq.shape
    Ck = ck.shape[2]
    est = np.zeros((B, H, Cq, Ck), np.float64)
    lib().orc_cluster_mass(cq, _c(nq, np.int32), ck, _c(nk, np.int32), B, H, Cq, Ck, D, float(scale), est)
    return est


def cluster_blocks(crow_ptr, ccol_idx, qoff, koff, NB):
    """Block CSR (row_ptr [B*H*NB + 1], col_idx) of a cluster CSR."""
    qoff, koff = _c(qoff, np.int32), _c(koff, np.int32)
    B, H, Cq1 = qoff.shape
    Ck = koff.shape[2] - 1
    row_ptr = np.zeros(B * H * NB + 1, np.int32)
    col_idx = np.zeros(max(B * H * NB * NB, 1), np.int32)
    ci = _c(ccol_idx, np.int32) if len(ccol_idx) else np.zeros(1, np.int32)
    nnz = lib().orc_cluster_blocks(_c(crow_ptr, np.int32), ci, qoff, koff, B, H, Cq1 - 1, Ck, int(NB),
                                   row_ptr, col_idx)
    return row_ptr, col_idx[:nnz].copy()


def cluster_attention(q, k, v, qassign, kassign, Cq, Ck, scale, crow_ptr, ccol_idx, tokens=None):
    """Raster output [B, N, H, D] float64 of attention under a cluster selection, or
    [B, H, len(tokens), D] for the listed query tokens only."""
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    B, N, H, D = q.shape
    tk = None if tokens is None else _c(tokens, np.int32)
    out = np.zeros((B, N, H, D) if tk is None else (B, H, len(tk), D), np.float64)
    ci = _c(ccol_idx, np.int32) if len(ccol_idx) else np.zeros(1, np.int32)
    lib().orc_cluster_attention(q, k, v, B, N, H, D, _c(qassign, np.int32), _c(kassign, np.int32), int(Cq),
                                int(Ck), float(scale), _c(crow_ptr, np.int32), ci,
                                None if tk is None else tk.ctypes.data, 0 if tk is None else len(tk), out)
    return out
