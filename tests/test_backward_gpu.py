"""GPU parity of the block-sparse backward and the CSR transpose against the CPU
oracle (gradients of masked attention written from the chain rule, in float64).
All calls go through the C ABI of libfpsa.so."""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_reorder_amd import fpsa, synth
from block_sparse_attention_reorder_amd.pipeline import BlockSparseAttention, Csr
from block_sparse_attention_reorder_amd.workloads import WORKLOADS

from parity_util import csr_to_numpy, dev, expected_tiled_rows, inputs, rows_to_qk

pytestmark = pytest.mark.gpu

# Gradient tolerances. Every gradient element is a sum of terms (scale ds_ij k_jd over
# keys for dq, scale ds_ij q_id over queries for dk, p_ij dO_id for dv). The oracle
# returns per element mag = the sum of |term| plus, for dq and dk, the term scale
# p_ij a_i/4 |k_jd| (or |q_id|), a_i = sum_d |dO_id| sum_j p_ij |v_jd| being how far
# delta_i = dO_i.o_i moves per unit relative error of o_i. Error sources: rounding p
# or ds to bf16 before each product (2^-9 of each term), p's relative error through
# the forward's lse (its normaliser sums bf16-rounded probabilities, about 2^-9), the
# bf16 storage of the result (2^-9 of |want| <= mag), and delta_i taken from the
# forward's float32 output, whose probabilities were rounded (at most about 2^-8
# a_i, i.e. 2^-6 of the a_i/4 part). The bound is |err| <= MAG_BOUND mag with
# MAG_BOUND = 2^-6 = 8 x 2^-9. Taking delta from the bf16 output adds 2^-9 a_i, hence
# BF16_O_FACTOR. The mean error must also stay below MEAN x rms(want); with delta from
# the bf16 output that error is systematic per query and the mean of dq and dk's
# errors grows to about 0.7 % of rms (MEAN_BF16_O).
MAG_BOUND = 2.0 ** -6
MEAN = 3e-3
BF16_O_FACTOR = 2.0
MEAN_BF16_O = 1e-2


def _dout(grid, B, H, D, seed):
    N = grid[0] * grid[1] * grid[2]
    g = np.random.default_rng(seed).standard_normal((B, N, H, D), dtype=np.float32)
    return synth.to_bf16_values(g)


def _gpu_grads(q, k, v, g, grid, tile, H, D, rp, ci, o_f32=True):
    bsa = BlockSparseAttention(grid, tile, 1, H, D)
    qt = bsa.tile_qk(dev(q, torch.bfloat16))
    kt = bsa.tile_qk(dev(k, torch.bfloat16))
    vt = bsa.tile_vt(dev(v, torch.bfloat16))
    vq = bsa.tile_qk(dev(v, torch.bfloat16))
    gt = bsa.tile_qk(dev(g, torch.bfloat16))
    csr = Csr(dev(rp, torch.int32), dev(ci if len(ci) else np.zeros(1, np.int32), torch.int32))
    lse = torch.empty((1, H, bsa.npad), dtype=torch.float32, device="cuda")
    o32 = torch.empty(bsa.tiled_shape(), dtype=torch.float32, device="cuda") if o_f32 else None
    ot = bsa.forward(qt, kt, vt, csr, lse=lse, out_f32=o32)
    csc = bsa.transpose(csr)
    dq, dk, dv = bsa.backward(qt, kt, vq, o32 if o_f32 else ot, gt, lse, csr, csc)
    raster = [bsa.untile(x, torch.float32).cpu().numpy() for x in (dq, dk, dv)]
    tiled = [x.float().cpu().numpy() for x in (dq, dk, dv)]
    return bsa, raster, tiled


def _check(got, want, mag, name, loose=1.0, mean=None):
    mean = MEAN if mean is None else mean
    rms = float(np.sqrt(np.mean(np.square(want))))
    err = np.abs(got.astype(np.float64) - want)
    worst = float((err / (loose * MAG_BOUND * mag + 1e-6 * rms)).max())
    print(f"{name}: err / bound {worst:.3f}, mean err / rms {err.mean() / rms:.5f}")
    assert worst <= 1.0 and err.mean() <= mean * rms, (name, worst, err.mean() / rms)


def _csr_of_rows(H, nb, seed, num, den, empty=()):
    m = synth.random_mass_rows(H * nb, nb, seed=seed, tie_frac=0.1, zero_frac=0.2)
    for r in empty:
        m[r] = 0.0
    return O.select_blocks(m, num, den)


# --------------------------------------------------------------------------- transpose

@pytest.mark.parametrize("B,H,nb", [(1, 1, 1), (1, 2, 5), (2, 3, 40), (1, 2, 200), (1, 1, 1440)])
def test_csr_transpose_bitexact(B, H, nb):
    R = B * H * nb
    rp, ci = _csr_of_rows(B * H, nb, R + nb, 1, 2)
    if R > 3:
        # a row with repeats and out-of-range indices
        extra = np.array([-1, 0, 0, nb, nb + 7, nb - 1], np.int32)
        ci = np.concatenate([ci[:rp[2]], extra, ci[rp[2]:]]).astype(np.int32)
        rp = rp.copy()
        rp[2:] += len(extra)
    bsa_csr = Csr(dev(rp, torch.int32), dev(ci, torch.int32))
    cp = torch.empty(R + 1, dtype=torch.int32, device="cuda")
    ri = torch.full((R * nb,), -5, dtype=torch.int32, device="cuda")
    ws = torch.empty(fpsa.transpose_workspace_bytes(R, nb), dtype=torch.uint8, device="cuda")
    fpsa.csr_transpose(bsa_csr.row_ptr, bsa_csr.col_idx, B, H, nb, cp, ri, ws)
    cp_g, ri_g = csr_to_numpy(cp, ri)
    cp_o, ri_o = O.csr_transpose(rp, ci, B, H, nb)
    assert np.array_equal(cp_g, cp_o) and np.array_equal(ri_g, ri_o)


# --------------------------------------------------------------------------- gradients

BWD_CASES = [((4, 8, 8), 1, 64), ((5, 6, 7), 2, 128), ((9, 10, 13), 2, 64), ((6, 9, 14), 2, 128)]


@pytest.mark.parametrize("grid,H,D", BWD_CASES)
@pytest.mark.parametrize("num,den", [(1, 2), (99, 100)])
@pytest.mark.parametrize("o_f32", [True, False])
def test_backward_matches_oracle(grid, H, D, num, den, o_f32):
    tile = (4, 4, 4)
    q, k, v = inputs(grid, 1, H, D, amp=1.5, seed=51)
    g = _dout(grid, 1, H, D, 52)
    nb = O.num_blocks(grid, tile)
    rp, ci = _csr_of_rows(H, nb, nb + 3 * H, num, den, empty=(0,))
    bsa, (dq, dk, dv), tiled = _gpu_grads(q, k, v, g, grid, tile, H, D, rp, ci, o_f32=o_f32)
    wq, wk, wv, mq, mk, mv = O.masked_attention_bwd(q, k, v, g, grid, tile, bsa.scale, rp, ci, magnitudes=True)
    loose, mean = (1.0, MEAN) if o_f32 else (BF16_O_FACTOR, MEAN_BF16_O)
    _check(dq, wq, mq, "dq", loose, mean)
    _check(dk, wk, mk, "dk", loose, mean)
    _check(dv, wv, mv, "dv")
    # the query block without kept keys gets exactly zero dq; padding rows of every
    # tiled gradient are exactly zero
    blk, slot = O.token_blocks(grid, tile)
    assert np.all(dq[0, blk == 0, 0] == 0)
    pad = np.setdiff1d(np.arange(bsa.npad), slot)
    for t in tiled:
        assert np.all(t[:, :, pad, :] == 0)


def test_backward_all_blocks_equals_dense_gradients():
    grid, tile, H, D = (5, 6, 7), (4, 4, 4), 2, 128
    q, k, v = inputs(grid, 1, H, D, amp=1.0, seed=53)
    g = _dout(grid, 1, H, D, 54)
    nb = O.num_blocks(grid, tile)
    rp = np.arange(0, H * nb * nb + 1, nb, dtype=np.int32)
    ci = np.tile(np.arange(nb, dtype=np.int32), H * nb)
    bsa, (dq, dk, dv), _ = _gpu_grads(q, k, v, g, grid, tile, H, D, rp, ci)
    wq, wk, wv, mq, mk, mv = O.masked_attention_bwd(q, k, v, g, grid, tile, bsa.scale, rp, ci, magnitudes=True)
    _check(dq, wq, mq, "dq")
    _check(dk, wk, mk, "dk")
    _check(dv, wv, mv, "dv")


def test_backward_odd_block_count_and_untidy_rows():
    """D = 128 on a video grid of 15 blocks (the last two-block workgroup of the dQ pass
    holds one query block; the last query block keeps nothing). Rows shuffled, with
    repeated and out-of-range entries: every gradient bit-identical to that of the same
    rows sorted and cleaned (repeats count once and out-of-range entries drop out, in
    the forward, the transpose and both gradient passes), and within the bounds of the
    oracle under the cleaned rows."""
    grid, tile, H, D = (4, 12, 20), (4, 4, 4), 2, 128
    q, k, v = inputs(grid, 1, H, D, amp=1.5, seed=57)
    g = _dout(grid, 1, H, D, 58)
    nb = O.num_blocks(grid, tile)
    assert nb % 2 == 1
    rp, ci = _csr_of_rows(H, nb, 11, 9, 10, empty=(H * nb - 1,))
    rng = np.random.default_rng(5)
    rows_bad = []
    for r in range(H * nb):
        row = ci[rp[r]:rp[r + 1]].tolist()
        bad = row + row[: len(row) // 3] + [nb, -1, 1 << 20][: r % 3]
        rng.shuffle(bad)
        rows_bad.append(bad)
    rp_bad = np.concatenate([[0], np.cumsum([len(x) for x in rows_bad])]).astype(np.int32)
    ci_bad = np.array([x for row in rows_bad for x in row], np.int32)
    bsa, raster, tiled = _gpu_grads(q, k, v, g, grid, tile, H, D, rp, ci)
    _, _, tiled_bad = _gpu_grads(q, k, v, g, grid, tile, H, D, rp_bad, ci_bad)
    for a, b in zip(tiled, tiled_bad):
        assert np.array_equal(a, b)
    wq, wk, wv, mq, mk, mv = O.masked_attention_bwd(q, k, v, g, grid, tile, bsa.scale, rp, ci, magnitudes=True)
    dq, dk, dv = raster
    _check(dq, wq, mq, "dq")
    _check(dk, wk, mk, "dk")
    _check(dv, wv, mv, "dv")
    blk, _ = O.token_blocks(grid, tile)
    assert np.all(dq[0, blk == nb - 1, H - 1] == 0)


def test_backward_repeat_is_bitwise_identical():
    grid, tile, H, D = (9, 10, 13), (4, 4, 4), 2, 128
    q, k, v = inputs(grid, 1, H, D, seed=55)
    g = _dout(grid, 1, H, D, 56)
    nb = O.num_blocks(grid, tile)
    rp, ci = _csr_of_rows(H, nb, 9, 99, 100)
    _, _, t1 = _gpu_grads(q, k, v, g, grid, tile, H, D, rp, ci)
    _, _, t2 = _gpu_grads(q, k, v, g, grid, tile, H, D, rp, ci)
    for a, b in zip(t1, t2):
        assert np.array_equal(a, b)


def test_backward_full_480p_sampled():
    """The full 480p path (mass pass, 99 % selection, forward, transpose, backward):
    dq of sampled query blocks of sampled heads against the oracle; for every head,
    the key gradients sum to zero over keys and the value gradients sum to the
    upstream gradient of the queries that attend anything (identities of the
    softmax backward), within the rounding of the stored bf16 gradients."""
    w = WORKLOADS["wan480p"]
    q, k, v = synth.make_qkv(w.grid, w.B, w.H, w.D, w.amp, w.sigma, w.seed, bf16=True)
    g = _dout(w.grid, w.B, w.H, w.D, 57)
    bsa = BlockSparseAttention(w.grid, w.tile, w.B, w.H, w.D)
    qd, kd, vd, gd = (torch.from_numpy(x).to("cuda").to(torch.bfloat16) for x in (q, k, v, g))
    qt, kt, vt, vq, gt = bsa.tile_qk(qd), bsa.tile_qk(kd), bsa.tile_vt(vd), bsa.tile_qk(vd), bsa.tile_qk(gd)
    csr = bsa.select(bsa.block_mass(qt, kt))
    lse = torch.empty((w.B, w.H, bsa.npad), dtype=torch.float32, device="cuda")
    o32 = torch.empty(bsa.tiled_shape(), dtype=torch.float32, device="cuda")
    bsa.forward(qt, kt, vt, csr, lse=lse, out_f32=o32)
    csc = bsa.transpose(csr)
    dq, dk, dv = (bsa.untile(x, torch.float32) for x in bsa.backward(qt, kt, vq, o32, gt, lse, csr, csc))
    torch.cuda.synchronize()
    rp, ci = csr_to_numpy(csr.row_ptr, csr.col_idx)
    dq = dq.cpu().numpy()
    # dq of sampled blocks: the oracle on the GPU's CSR rows would take HIP output as
    # oracle input, so the oracle selects on its own masses of those rows
    for h in (0, 11):
        blocks = [0, 311, bsa.nb - 1]
        qh, kh, vh, gh = (np.ascontiguousarray(x[:, :, h:h + 1]) for x in (q, k, v, g))
        mo = O.block_mass(qh, kh, w.grid, w.tile, bsa.scale, qblocks=blocks)[0, 0]
        rp_o, ci_o = O.select_blocks(mo.astype(np.float32))
        full_rp = np.zeros(bsa.nb + 1, np.int32)
        cnt = np.zeros(bsa.nb, np.int64)
        for i, b in enumerate(blocks):
            cnt[b] = rp_o[i + 1] - rp_o[i]
        full_rp[1:] = np.cumsum(cnt)
        same = [np.array_equal(ci[rp[h * bsa.nb + b]:rp[h * bsa.nb + b + 1]], ci_o[rp_o[i]:rp_o[i + 1]])
                for i, b in enumerate(blocks)]
        wq, mq, tok = O.masked_attention_bwd_dq(qh, kh, vh, gh, w.grid, w.tile, bsa.scale, full_rp, ci_o, blocks,
                                                magnitudes=True)
        for i, b in enumerate(blocks):
            if not same[i]:
                continue
            t = tok[0, 0, i][tok[0, 0, i] >= 0]
            _check(dq[0, t, h], wq[0, 0, i, :len(t)], mq[0, 0, i, :len(t)], f"dq head {h} block {b}")
    # identities over all keys of every head (float64 sums of the stored bf16 values)
    dk64 = dk.double().sum(dim=1).cpu().numpy()[0]               # [H, D]
    dv64 = dv.double().sum(dim=1).cpu().numpy()[0]
    dk_abs = dk.double().abs().sum(dim=1).cpu().numpy()[0]
    dv_abs = dv.double().abs().sum(dim=1).cpu().numpy()[0]
    blk, _ = O.token_blocks(w.grid, w.tile)
    cnt = np.diff(rp).reshape(w.H, bsa.nb)
    worst_k = worst_v = 0.0
    for h in range(w.H):
        live = cnt[h][blk] > 0
        want_v = g[0, live, h].astype(np.float64).sum(axis=0)
        worst_k = max(worst_k, float((np.abs(dk64[h]) / dk_abs[h]).max()))
        worst_v = max(worst_v, float((np.abs(dv64[h] - want_v) / dv_abs[h]).max()))
    print(f"key-sum identities: |sum dk| / sum |dk| <= {worst_k:.3e}, |sum dv - sum dO| / sum |dv| <= {worst_v:.3e}")
    # each stored element carries a bf16 rounding (2^-9 of itself) on top of terms
    # rounded by as much: the sums stay within 2^-8 of the sum of magnitudes
    assert worst_k <= 2.0 ** -8 and worst_v <= 2.0 ** -8


# --------------------------------------------------------------------------- FP8

@pytest.mark.parametrize("grid,H,D", [((5, 6, 7), 2, 128), ((9, 10, 13), 2, 64)])
def test_dequantize_tiles_bitexact(grid, H, D):
    tile = (4, 4, 4)
    q = inputs(grid, 2, H, D, amp=2.0, seed=71)[0]
    bsa = BlockSparseAttention(grid, tile, 2, H, D)
    q8, qs = bsa.tile_fp8(dev(q, torch.bfloat16))
    got = bsa.dequantize(q8, qs).view(torch.int16).cpu().numpy()
    rows = expected_tiled_rows(O.fp8_dequantized_bf16(q, grid, tile), grid, tile)
    want = rows_to_qk(torch.from_numpy(rows).to(torch.bfloat16).view(torch.int16).numpy(), bsa.nb, esize=2)
    assert np.array_equal(got.reshape(want.shape), want)
    # without a scale: the code values themselves, exact in bf16
    codes, _ = O.fp8_tile_codes(q, grid, tile)
    vals = np.vectorize(O.e4m3_decode)(codes).astype(np.float32)
    got = bsa.dequantize(q8, None).view(torch.int16).cpu().numpy()
    rows = expected_tiled_rows(vals, grid, tile)
    want = rows_to_qk(torch.from_numpy(rows).to(torch.bfloat16).view(torch.int16).numpy(), bsa.nb, esize=2)
    assert np.array_equal(got.reshape(want.shape), want)


# The backward of the FP8 forward: the gradient of attention at the dequantized Q and K
# (the quantizer passes gradients straight through). The kernels read the e4m3 code
# values as bf16 (exact) with the tile scales, so their scores are the forward's and
# the only new rounding is that of ds times the tile scale before the dq and dk
# products, inside the bf16 bounds above.


@pytest.mark.parametrize("grid,H,D", [((5, 6, 7), 2, 128), ((9, 10, 13), 2, 64), ((6, 9, 14), 1, 128),
                                      ((12, 20, 24), 1, 64)])
def test_fp8_backward_matches_oracle(grid, H, D):
    tile = (4, 4, 4)
    q, k, v = inputs(grid, 1, H, D, amp=1.5, seed=73)
    g = _dout(grid, 1, H, D, 74)
    nb = O.num_blocks(grid, tile)
    if nb > 64:
        # flat rows keep nearly every block, so the key tile scales of a row come from
        # several 64-entry windows (and the columns are as long)
        m = np.random.default_rng(nb).random((H * nb, nb)).astype(np.float32)
        rp, ci = O.select_blocks(m / m.sum(axis=1, keepdims=True), 99, 100)
        assert np.diff(rp).min() > 64
    else:
        rp, ci = _csr_of_rows(H, nb, nb + 5 * H, 99, 100, empty=(0,))
    bsa = BlockSparseAttention(grid, tile, 1, H, D)
    q8, qs = bsa.tile_fp8(dev(q, torch.bfloat16))
    k8, ks = bsa.tile_fp8(dev(k, torch.bfloat16))
    vt = bsa.tile_vt(dev(v, torch.bfloat16))
    vq = bsa.tile_qk(dev(v, torch.bfloat16))
    gt = bsa.tile_qk(dev(g, torch.bfloat16))
    csr = Csr(dev(rp, torch.int32), dev(ci if len(ci) else np.zeros(1, np.int32), torch.int32))
    lse = torch.empty((1, H, bsa.npad), dtype=torch.float32, device="cuda")
    o32 = torch.empty(bsa.tiled_shape(), dtype=torch.float32, device="cuda")
    bsa.forward(q8, k8, vt, csr, q_scale=qs, k_scale=ks, lse=lse, out_f32=o32)
    qc, kc = bsa.dequantize(q8, None), bsa.dequantize(k8, None)
    csc = bsa.transpose(csr)
    grads = bsa.backward(qc, kc, vq, o32, gt, lse, csr, csc, q_scale=qs, k_scale=ks)
    dq, dk, dv = (bsa.untile(x, torch.float32).cpu().numpy() for x in grads)
    xq, _ = O.fp8_tile_quantize(q, grid, tile)
    xk, _ = O.fp8_tile_quantize(k, grid, tile)
    wq, wk, wv, mq, mk, mv = O.masked_attention_bwd(xq, xk, v, g, grid, tile, bsa.scale, rp, ci, magnitudes=True)
    _check(dq, wq, mq, "dq")
    _check(dk, wk, mk, "dk")
    _check(dv, wv, mv, "dv")
