"""GPU parity of the k-means semantic permutation (clusters, layout, gathers, cluster
masses, cluster selection, block CSR, forward over counted blocks) against the CPU
oracle. All calls go through the C ABI of libfpsa.so."""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_reorder_amd import fpsa, synth
from block_sparse_attention_reorder_amd.pipeline import SemanticSparseAttention
from block_sparse_attention_reorder_amd.workloads import WORKLOADS

from parity_util import BF16_MAX_ABS, BF16_MEAN_ABS, csr_to_numpy, dev, rows_to_qk, rows_to_vt

pytestmark = pytest.mark.gpu

# grid (token count and structure of the inputs), heads, head size, query and key
# clusters, k-means steps
CASES = [((4, 8, 8), 2, 64, 7, 5, 3), ((5, 6, 7), 2, 128, 16, 12, 4), ((9, 10, 13), 1, 128, 32, 24, 6),
         ((6, 9, 14), 2, 64, 40, 40, 5)]


def _inputs(grid, H, D, seed, amp=1.5):
    return synth.make_qkv(grid, 1, H, D, amp, 1.0, seed, bf16=True)


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("f32", [False, True])
def test_kmeans_and_layout_bitexact(case, f32):
    grid, H, D, Cq, _, iters = case
    q, _, _ = _inputs(grid, H, D, 61)
    N = q.shape[1]
    ssa = SemanticSparseAttention(N, 1, H, D, Cq, Cq, iters=iters)
    c = ssa.cluster(dev(q, torch.float32 if f32 else torch.bfloat16), Cq)
    a, cent, cnt = O.kmeans(q, Cq, iters)
    assert np.array_equal(c.assign.cpu().numpy(), a)
    assert np.array_equal(c.counts.cpu().numpy(), cnt)
    assert np.array_equal(c.centroids.cpu().numpy(), cent)          # bit for bit in float64
    mo = c.member_off.cpu().numpy()
    mem = c.members.cpu().numpy()
    for h in range(H):
        for k in range(Cq):
            r = h * Cq + k
            assert np.array_equal(mem[mo[r]:mo[r + 1]], np.where(a[0, h] == k)[0])
    st, off, bc = O.cluster_layout(a, Cq, ssa.NB)
    assert np.array_equal(c.slot_token.cpu().numpy(), st)
    assert np.array_equal(c.blk_off.cpu().numpy(), off)
    assert np.array_equal(c.blk_count.cpu().numpy(), bc)


@pytest.mark.parametrize("N,H,D,C,iters", [(33, 2, 64, 1, 3), (33, 1, 128, 33, 2), (700, 2, 64, 300, 3),
                                           (1030, 1, 128, 129, 2)])
def test_kmeans_extreme_cluster_counts(N, H, D, C, iters):
    """One cluster; as many clusters as tokens (every token starts as its own
    centroid); cluster counts that leave a partial last centroid tile; token counts
    that leave a partial last workgroup."""
    rng = np.random.default_rng(N + C)
    x = (rng.standard_normal((1, N, H, D)) * 2.0).astype(np.float32)
    xb = dev(x, torch.bfloat16)
    xr = xb.float().cpu().numpy()                   # the bf16 values, exactly
    i32 = dict(dtype=torch.int32, device="cuda")
    a, cnt = torch.empty((1, H, N), **i32), torch.empty((1, H, C), **i32)
    cent = torch.empty((1, H, C, D), dtype=torch.float64, device="cuda")
    mo, mem = torch.empty(H * C + 1, **i32), torch.empty(H * N, **i32)
    ws = torch.empty(fpsa.kmeans_workspace_bytes(1, H, N, C), dtype=torch.uint8, device="cuda")
    fpsa.kmeans(xb, 1, N, H, D, C, iters, a, cent, cnt, mo, mem, ws)
    ra, rc, rn = O.kmeans(xr, C, iters)
    assert np.array_equal(a.cpu().numpy(), ra)
    assert np.array_equal(cnt.cpu().numpy(), rn)
    assert np.array_equal(cent.cpu().numpy(), rc)


@pytest.mark.parametrize("D", [64, 128])
def test_gather_and_scatter_by_slot_map(D):
    grid, H, C = (5, 6, 7), 2, 9
    q, _, _ = _inputs(grid, H, D, 62)
    N = q.shape[1]
    a, _, _ = O.kmeans(q, C, 2)
    NB = O.blocks_for(N, C)
    st, _, _ = O.cluster_layout(a, C, NB)
    qd, std = dev(q, torch.bfloat16), dev(st, torch.int32)
    # expected tiled rows from the slot map, then the operand layouts of the header
    rows = np.zeros((1, H, NB * 64, D), np.float32)
    for h in range(H):
        real = st[0, h] >= 0
        rows[0, h, real] = q[0, st[0, h][real], h]
    rows_bits = torch.from_numpy(rows).to(torch.bfloat16).view(torch.int16).numpy()
    for layout, want in ((fpsa.LAYOUT_ROWS, rows_bits.reshape(1, H, NB, 64 * D)),
                         (fpsa.LAYOUT_QK, rows_to_qk(rows_bits, NB)), (fpsa.LAYOUT_VT, rows_to_vt(rows_bits, NB))):
        out = torch.empty((1, H, NB * 64, D), dtype=torch.bfloat16, device="cuda")
        fpsa.gather_tiles(qd, std, 1, N, H, D, NB, layout, out)
        got = out.view(torch.int16).cpu().numpy().reshape(1, H, NB, 64 * D)
        assert np.array_equal(got, want.reshape(1, H, NB, 64 * D)), layout
    rows_t = torch.empty((1, H, NB * 64, D), dtype=torch.bfloat16, device="cuda")
    fpsa.gather_tiles(qd, std, 1, N, H, D, NB, fpsa.LAYOUT_ROWS, rows_t)
    back = torch.full((1, N, H, D), 7.0, dtype=torch.float32, device="cuda")
    fpsa.scatter_tiles(rows_t, std, 1, N, H, D, NB, back)
    assert np.array_equal(back.cpu().numpy(), q)                  # q holds bf16 values


@pytest.mark.parametrize("case", CASES)
def test_cluster_mass_selection_and_blocks(case):
    grid, H, D, Cq, Ck, iters = case
    q, k, _ = _inputs(grid, H, D, 63)
    N = q.shape[1]
    ssa = SemanticSparseAttention(N, 1, H, D, Cq, Ck, iters=iters)
    qa, qcent, qcnt = O.kmeans(q, Cq, iters)
    ka, kcent, kcnt = O.kmeans(k, Ck, iters)
    est_o = O.cluster_mass(qcent, qcnt, kcent, kcnt, np.float32(ssa.scale))
    est = torch.empty((1, H, Cq, Ck), dtype=torch.float32, device="cuda")
    fpsa.cluster_mass(dev(qcent, torch.float64), dev(qcnt, torch.int32), dev(kcent, torch.float64),
                      dev(kcnt, torch.int32), 1, H, Cq, Ck, D, ssa.scale, est)
    got = est.cpu().numpy()
    want = est_o.astype(np.float32)
    # float64 exponentials and sums in another order: the float32 results agree to an ulp
    assert np.all(np.abs(got - want) <= np.spacing(want)), np.abs(got - want).max()
    # selection of the oracle's (float32) masses: exact
    rows = want.reshape(-1, Ck)
    crp_o, cci_o = O.select_blocks(rows, *ssa.thr)
    ccsr = ssa.select_clusters(dev(rows, torch.float32))
    crp, cci = csr_to_numpy(ccsr.row_ptr, ccsr.col_idx)
    assert np.array_equal(crp, crp_o) and np.array_equal(cci, cci_o)
    # block CSR of the oracle's cluster selection and layout: exact
    _, qoff, _ = O.cluster_layout(qa, Cq, ssa.NB)
    _, koff, _ = O.cluster_layout(ka, Ck, ssa.NB)
    rp_o, ci_o = O.cluster_blocks(crp_o, cci_o, qoff, koff, ssa.NB)
    R = H * ssa.NB
    rp = torch.empty(R + 1, dtype=torch.int32, device="cuda")
    ci = torch.full((R * ssa.NB,), -3, dtype=torch.int32, device="cuda")
    fpsa.cluster_blocks(dev(crp_o, torch.int32), dev(cci_o if len(cci_o) else np.zeros(1, np.int32), torch.int32),
                        dev(qoff, torch.int32), dev(koff, torch.int32), 1, H, Cq, Ck, ssa.NB, rp, ci,
                        torch.empty(R, dtype=torch.int32, device="cuda"))
    rp_g, ci_g = csr_to_numpy(rp, ci)
    assert np.array_equal(rp_g, rp_o) and np.array_equal(ci_g, ci_o)


def _oracle_semantic(q, k, v, ssa):
    qa, qcent, qcnt = O.kmeans(q, ssa.Cq, ssa.iters)
    ka, kcent, kcnt = O.kmeans(k, ssa.Ck, ssa.iters)
    est = O.cluster_mass(qcent, qcnt, kcent, kcnt, np.float32(ssa.scale)).astype(np.float32)
    crp, cci = O.select_blocks(est.reshape(-1, ssa.Ck), *ssa.thr)
    return qa, ka, est, crp, cci


def _certify(same, rows, ssa):
    """A cluster row may differ from the oracle's only when its cut is fragile: the
    float32 masses agree to an ulp each, so its cut margin must be within the sum of
    its masses' ulps (twice, for both sides)."""
    if same.all():
        return
    bad = rows[~same].astype(np.float64)
    margin = O.cut_margin(bad, ssa.thr[0] / ssa.thr[1])
    assert np.all(margin <= 2 * np.spacing(rows[~same]).sum(axis=1)), margin


def _rows_equal(crp_a, cci_a, crp_b, cci_b):
    return np.array([np.array_equal(cci_a[crp_a[r]:crp_a[r + 1]], cci_b[crp_b[r]:crp_b[r + 1]])
                     for r in range(len(crp_a) - 1)])


@pytest.mark.parametrize("case", CASES)
def test_semantic_attention_end_to_end(case):
    grid, H, D, Cq, Ck, iters = case
    q, k, v = _inputs(grid, H, D, 64)
    N = q.shape[1]
    ssa = SemanticSparseAttention(N, 1, H, D, Cq, Ck, iters=iters)
    o, res = ssa.run(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), torch.float32)
    o = o.cpu().numpy()
    qa, ka, est, crp, cci = _oracle_semantic(q, k, v, ssa)
    assert np.array_equal(res["qc"].assign.cpu().numpy(), qa)
    assert np.array_equal(res["kc"].assign.cpu().numpy(), ka)
    crp_g, cci_g = csr_to_numpy(res["ccsr"].row_ptr, res["ccsr"].col_idx)
    same = _rows_equal(crp_g, cci_g, crp, cci)
    _certify(same, est.reshape(-1, Ck), ssa)
    ref = O.cluster_attention(q, k, v, qa, ka, Cq, Ck, ssa.scale, crp, cci)
    errs = []
    for h in range(H):
        ok = same[h * Cq + qa[0, h]]                    # queries whose cluster row matched
        errs.append(np.abs(o[0, ok, h].astype(np.float64) - ref[0, ok, h]).ravel())
    e = np.concatenate(errs)
    assert e.max() <= BF16_MAX_ABS and e.mean() <= BF16_MEAN_ABS, (e.max(), e.mean())


def test_semantic_full_480p_sampled():
    """The 480p shape with 128 query and 128 key clusters: every cluster of heads 0 and
    11 bit-exact against the oracle's k-means, their cluster masses within an ulp, and
    outputs of sampled query tokens against attention under the oracle's selection."""
    w = WORKLOADS["wan480p"]
    q, k, v = synth.make_qkv(w.grid, w.B, w.H, w.D, w.amp, w.sigma, w.seed, bf16=True)
    N = q.shape[1]
    ssa = SemanticSparseAttention(N, w.B, w.H, w.D, 128, 128, iters=4)
    o, res = ssa.run(*(torch.from_numpy(x).to("cuda").to(torch.bfloat16) for x in (q, k, v)), torch.float32)
    o = o.cpu().numpy()
    est_g = res["est"].cpu().numpy()
    crp_g, cci_g = csr_to_numpy(res["ccsr"].row_ptr, res["ccsr"].col_idx)
    rng = np.random.default_rng(7)
    for h in (0, 11):
        qh, kh, vh = (np.ascontiguousarray(x[:, :, h:h + 1]) for x in (q, k, v))
        qa, ka, est, crp, cci = _oracle_semantic(qh, kh, vh, ssa)
        assert np.array_equal(res["qc"].assign.cpu().numpy()[:, h:h + 1], qa)
        assert np.array_equal(res["kc"].assign.cpu().numpy()[:, h:h + 1], ka)
        assert np.all(np.abs(est_g[:, h:h + 1] - est) <= np.spacing(est))
        rows = slice(h * ssa.Cq, (h + 1) * ssa.Cq)
        sub_rp = crp_g[rows.start:rows.stop + 1] - crp_g[rows.start]
        sub_ci = cci_g[crp_g[rows.start]:crp_g[rows.stop]]
        same = _rows_equal(sub_rp, sub_ci, crp, cci)
        _certify(same, est.reshape(-1, ssa.Ck), ssa)
        toks = np.sort(rng.choice(N, size=48, replace=False)).astype(np.int32)
        toks = toks[same[qa[0, 0, toks]]]
        ref = O.cluster_attention(qh, kh, vh, qa, ka, ssa.Cq, ssa.Ck, ssa.scale, crp, cci, tokens=toks)
        e = np.abs(o[0, toks, h].astype(np.float64) - ref[0, 0])
        assert e.max() <= BF16_MAX_ABS and e.mean() <= BF16_MEAN_ABS, (h, e.max(), e.mean())
