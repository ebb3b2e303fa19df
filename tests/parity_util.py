"""Shared helpers for the GPU parity tests (inputs, layouts, comparisons).

Expected values come only from the CPU oracle or from the layout definitions in
include/fpsa.h; nothing here is computed by the HIP path.
"""
import numpy as np
import torch

import oracle as O
from block_sparse_attention_reorder_amd import synth

# P*V operand order inside each run of 16 keys, as documented for the VT layout.
VT_RUN_ORDER = [0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15]

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
FP8_MAX_ABS = 6e-2


def value_scale(v):
    """Output tolerances scale with the size of V: the bf16 rounding of the
    probabilities perturbs each output by a fraction of |v|. The stated bf16 bounds
    apply as written up to an rms |v| of 1.25 (the amp <= 1.5 workloads) and grow
    linearly beyond it (sharper test inputs with amp 3-4)."""
    return max(1.0, float(np.sqrt(np.mean(np.square(v, dtype=np.float64)))) / 1.25)


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype)


def inputs(grid, B, H, D, amp=1.0, sigma=1.0, seed=0, bf16=True):
    return synth.make_qkv(grid, B, H, D, amp, sigma, seed, bf16=bf16)


def expected_tiled_rows(x, grid, tile):
    """bf16-rounded tiled rows [B, H, Npad, D] (as float32) from raster x."""
    B, N, H, D = x.shape
    nb = O.num_blocks(grid, tile)
    _, slot = O.token_blocks(grid, tile)
    out = np.zeros((B, H, nb * 64, D), np.float32)
    xb = synth.to_bf16_values(x)
    out[:, :, slot, :] = np.transpose(xb, (0, 2, 1, 3))
    return out


def rows_to_vt(rows, nb):
    """tiled rows [B, H, Npad, D] -> VT layout, flat per block, following the header:
    element (e, d) at ((((d/32)*4 + P/16)*2 + (P/8)%2)*32 + d%32)*8 + P%8, where P is
    the position of slot e (runs of 16 ordered slots 0-3, 8-11, 4-7, 12-15)."""
    B, H, _, D = rows.shape
    blocks = rows.reshape(B, H, nb, 64, D)
    out = np.zeros((B, H, nb, 64 * D), rows.dtype)
    pos_of_slot = np.zeros(64, np.int64)
    for P in range(64):
        pos_of_slot[16 * (P // 16) + VT_RUN_ORDER[P % 16]] = P
    e = np.arange(64)[:, None]
    d = np.arange(D)[None, :]
    P = pos_of_slot[e]
    off = ((((d // 32) * 4 + P // 16) * 2 + (P // 8) % 2) * 32 + d % 32) * 8 + P % 8
    out[:, :, :, off.ravel()] = blocks.reshape(B, H, nb, 64 * D)
    return out


def rows_to_qk(rows, nb, esize=2):
    """tiled rows [B, H, Npad, D] -> QK layout, flat per block, following the header."""
    B, H, _, D = rows.shape
    blocks = rows.reshape(B, H, nb, 64, D)
    out = np.zeros((B, H, nb, 64 * D), rows.dtype)
    e = np.arange(64)[:, None]
    d = np.arange(D)[None, :]
    if esize == 2:
        off = ((((e // 32) * (D // 16) + d // 16) * 2 + (d // 8) % 2) * 32 + e % 32) * 8 + d % 8
    else:
        off = ((((e // 32) * (D // 64) + d // 64) * 2 + (d // 32) % 2) * 32 + e % 32) * 32 + d % 32
    out[:, :, :, off.ravel()] = blocks.reshape(B, H, nb, 64 * D)
    return out


def csr_to_numpy(row_ptr, col_idx):
    rp = row_ptr.cpu().numpy()
    ci = col_idx[: int(rp[-1])].cpu().numpy()
    return rp, ci


def csr_rows(rp, ci):
    return [ci[rp[r]:rp[r + 1]] for r in range(len(rp) - 1)]


def compare_selection(rp_gpu, ci_gpu, rp_orc, ci_orc, mass_orc64, mass_gpu):
    """Rows whose kept set differs; each must be certified fragile (oracle cut margin
    within twice the row's largest mass error). Returns (n_diff, n_uncertified)."""
    rows_g, rows_o = csr_rows(rp_gpu, ci_gpu), csr_rows(rp_orc, ci_orc)
    nb = mass_orc64.shape[-1]
    m64 = mass_orc64.reshape(-1, nb)
    mg = mass_gpu.reshape(-1, nb).astype(np.float64)
    diff = [r for r in range(len(rows_o)) if not np.array_equal(rows_g[r], rows_o[r])]
    if not diff:
        return 0, 0
    margin = O.cut_margin(m64[diff], 0.99)
    err = np.abs(mg[diff] - m64[diff]).max(axis=1)
    bad = int(np.sum(margin > 2 * err))
    return len(diff), bad


def scatter_oracle_rows(out, tok):
    """Yield (b, h, token, out_row) for every real token in an oracle masked output."""
    B, H, S, _ = tok.shape
    for b in range(B):
        for h in range(H):
            for s in range(S):
                t = tok[b, h, s]
                n = int((t >= 0).sum())
                yield b, h, t[:n], out[b, h, s, :n]


def output_errors(o_gpu_raster, out, tok):
    """(max abs, mean abs) of GPU raster output [B, N, H, D] vs oracle rows."""
    errs = []
    for b, h, t, ref in scatter_oracle_rows(out, tok):
        errs.append(np.abs(o_gpu_raster[b, t, h, :].astype(np.float64) - ref).ravel())
    e = np.concatenate(errs)
    return float(e.max()), float(e.mean())
