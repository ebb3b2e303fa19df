"""Batch size above one on the GPU: the tile moves, the mass pass, the selection, the
forward (bf16 and e4m3), the backward and the k-means permutation index every tensor
by (batch, head); each is compared with the CPU oracle on a two-sample batch whose
samples differ."""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_reorder_amd import synth
from block_sparse_attention_reorder_amd.pipeline import BlockSparseAttention, Csr, SemanticSparseAttention

from parity_util import BF16_MAX_ABS, BF16_MEAN_ABS, csr_to_numpy, dev, output_errors

pytestmark = pytest.mark.gpu

GRID, TILE, B, H, D = (5, 6, 7), (4, 4, 4), 2, 2, 128


def _inputs(seed=71):
    return synth.make_qkv(GRID, B, H, D, 1.5, 1.0, seed, bf16=True)


def test_batch_mass_selection_and_forward():
    q, k, v = _inputs()
    bsa = BlockSparseAttention(GRID, TILE, B, H, D)
    qt, kt = bsa.tile_qk(dev(q, torch.bfloat16)), bsa.tile_qk(dev(k, torch.bfloat16))
    vt = bsa.tile_vt(dev(v, torch.bfloat16))
    mass = bsa.block_mass(qt, kt)
    mo = O.block_mass(q, k, GRID, TILE, bsa.scale)
    mg = mass.cpu().numpy().astype(np.float64)
    assert np.abs(mg - mo).max() < 1e-6
    assert not np.allclose(mo[0], mo[1])                    # the two samples differ
    # selection of the oracle's masses through the GPU: exact, rows (b*H + h)*nb + qb
    csr = bsa.select(dev(mo.astype(np.float32), torch.float32), 1, 2)
    rp, ci = csr_to_numpy(csr.row_ptr, csr.col_idx)
    rp_o, ci_o = O.select_blocks(mo.astype(np.float32), 1, 2)
    assert np.array_equal(rp, rp_o) and np.array_equal(ci, ci_o)
    o = bsa.untile(bsa.forward(qt, kt, vt, csr), torch.float32).cpu().numpy()
    out, tok = O.masked_attention(q, k, v, GRID, TILE, bsa.scale, rp_o, ci_o)
    mx, mean = output_errors(o, out, tok)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)


def test_batch_fp8_forward():
    q, k, v = _inputs(72)
    bsa = BlockSparseAttention(GRID, TILE, B, H, D)
    nb = bsa.nb
    rp, ci = O.select_blocks(synth.random_mass_rows(B * H * nb, nb, seed=3), 9, 10)
    qt, qs = bsa.tile_fp8(dev(q, torch.bfloat16))
    kt, ks = bsa.tile_fp8(dev(k, torch.bfloat16))
    vt = bsa.tile_vt(dev(v, torch.bfloat16))
    csr = Csr(dev(rp, torch.int32), dev(ci, torch.int32))
    o = bsa.untile(bsa.forward(qt, kt, vt, csr, q_scale=qs, k_scale=ks), torch.float32).cpu().numpy()
    qh, _ = O.fp8_tile_quantize(q, GRID, TILE)
    kh, _ = O.fp8_tile_quantize(k, GRID, TILE)
    out, tok = O.masked_attention(qh, kh, v, GRID, TILE, bsa.scale, rp, ci)
    mx, mean = output_errors(o, out, tok)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)


def test_batch_backward():
    q, k, v = _inputs(73)
    g = synth.to_bf16_values(np.random.default_rng(74).standard_normal(q.shape, dtype=np.float32))
    bsa = BlockSparseAttention(GRID, TILE, B, H, D)
    nb = bsa.nb
    rp, ci = O.select_blocks(synth.random_mass_rows(B * H * nb, nb, seed=4), 9, 10)
    qt, kt = bsa.tile_qk(dev(q, torch.bfloat16)), bsa.tile_qk(dev(k, torch.bfloat16))
    vt, vq, gt = bsa.tile_vt(dev(v, torch.bfloat16)), bsa.tile_qk(dev(v, torch.bfloat16)), bsa.tile_qk(dev(g, torch.bfloat16))
    csr = Csr(dev(rp, torch.int32), dev(ci, torch.int32))
    lse = torch.empty((B, H, bsa.npad), dtype=torch.float32, device="cuda")
    o32 = torch.empty(bsa.tiled_shape(), dtype=torch.float32, device="cuda")
    bsa.forward(qt, kt, vt, csr, lse=lse, out_f32=o32)
    csc = bsa.transpose(csr)
    cp, cr = csr_to_numpy(csc.row_ptr, csc.col_idx)
    cp_o, cr_o = O.csr_transpose(rp, ci, B, H, nb)
    assert np.array_equal(cp, cp_o) and np.array_equal(cr, cr_o)
    grads = [bsa.untile(x, torch.float32).cpu().numpy() for x in bsa.backward(qt, kt, vq, o32, gt, lse, csr, csc)]
    want = O.masked_attention_bwd(q, k, v, g, GRID, TILE, bsa.scale, rp, ci, magnitudes=True)
    for got, w, mag in zip(grads, want[:3], want[3:]):
        err = np.abs(got.astype(np.float64) - w)
        assert np.all(err <= 2.0 ** -6 * mag + 1e-6), (err / (2.0 ** -6 * mag + 1e-6)).max()


def test_batch_semantic_permutation():
    q, k, v = _inputs(75)
    N = q.shape[1]
    ssa = SemanticSparseAttention(N, B, H, D, 9, 11, iters=3)
    o, res = ssa.run(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), torch.float32)
    qa, qc, qn = O.kmeans(q, 9, 3)
    ka, kc, kn = O.kmeans(k, 11, 3)
    assert np.array_equal(res["qc"].assign.cpu().numpy(), qa)
    assert np.array_equal(res["kc"].assign.cpu().numpy(), ka)
    assert np.array_equal(res["qc"].centroids.cpu().numpy(), qc)
    est = O.cluster_mass(qc, qn, kc, kn, np.float32(ssa.scale)).astype(np.float32)
    crp, cci = O.select_blocks(est.reshape(-1, 11), *ssa.thr)
    crp_g, cci_g = csr_to_numpy(res["ccsr"].row_ptr, res["ccsr"].col_idx)
    same = np.array([np.array_equal(cci_g[crp_g[r]:crp_g[r + 1]], cci[crp[r]:crp[r + 1]]) for r in range(B * H * 9)])
    rows = est.reshape(-1, 11)
    if not same.all():   # only rows whose cut lies within the masses' rounding may differ
        margin = O.cut_margin(rows[~same].astype(np.float64), ssa.thr[0] / ssa.thr[1])
        assert np.all(margin <= 2 * np.spacing(rows[~same]).sum(axis=1)), margin
    ref = O.cluster_attention(q, k, v, qa, ka, 9, 11, ssa.scale, crp, cci)
    og = o.cpu().numpy().astype(np.float64)
    errs = []
    for b in range(B):
        for h in range(H):
            ok = same[(b * H + h) * 9 + qa[b, h]]
            errs.append(np.abs(og[b, ok, h] - ref[b, ok, h]).ravel())
    e = np.concatenate(errs)
    assert e.max() <= BF16_MAX_ABS and e.mean() <= BF16_MEAN_ABS, (e.max(), e.mean())
