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


U64 = 2.0 ** -53


def _gamma(n):
    n = np.asarray(n, np.float64)
    return n * U64 / (1.0 - n * U64)


def _gpu_kmeans(xd, N, H, D, C, iters):
    i32 = dict(dtype=torch.int32, device="cuda")
    a, cnt = torch.empty((1, H, N), **i32), torch.empty((1, H, C), **i32)
    cent = torch.empty((1, H, C, D), dtype=torch.float64, device="cuda")
    mo, mem = torch.empty(H * C + 1, **i32), torch.empty(H * N, **i32)
    ws = torch.empty(fpsa.kmeans_workspace_bytes(1, H, N, C), dtype=torch.uint8, device="cuda")
    fpsa.kmeans(xd, 1, N, H, D, C, iters, a, cent, cnt, mo, mem, ws)
    return (a.cpu().numpy(), cent.cpu().numpy(), cnt.cpu().numpy(), mo.cpu().numpy(), mem.cpu().numpy())


def _check_kmeans(x, xd, C, iters):
    """The GPU's k-means against plain Lloyd in the oracle.

    Step by step (the GPU run for s steps against the GPU run for s - 1): every
    token's cluster is a nearest centroid of the previous centroids, exactly, except
    where two candidates lie within the certified float64 evaluation bound of each
    other (excess <= tol, either choice valid); counts and member lists are exact for
    that assignment; each centroid is the mean of its members within the rounding
    bound of any summation order, 2 gamma_n sum|x| / n plus a few ulps (the GPU sums
    members in eight interleaved partials, the oracle in token order).
    End to end: the assignment after the last step equals the oracle's own run."""
    N, H, D = x.shape[1], x.shape[2], x.shape[3]
    prev = O.kmeans_start(x, C)
    ulps = 0
    for s in range(1, iters + 1):
        a, cent, cnt, mo, mem = _gpu_kmeans(xd, N, H, D, C, s)
        _, excess, tol = O.kmeans_assign(x, prev, other=a)
        assert np.all(excess <= tol), (s, float((excess - tol).max()))
        ulps += int(np.sum(excess > 0))
        want, wcnt, abs_sum = O.kmeans_means(x, a, prev)
        assert np.array_equal(cnt, wcnt)
        n = np.maximum(wcnt, 1)[..., None].astype(np.float64)
        bound = 2 * _gamma(n) * abs_sum / n + 4 * U64 * np.abs(want)
        assert np.all(np.abs(cent - want) <= bound), (s, float((np.abs(cent - want) - bound).max()))
        for h in range(H):
            for k in range(C):
                r = h * C + k
                assert np.array_equal(mem[mo[r]:mo[r + 1]], np.where(a[0, h] == k)[0])
        prev = cent
    ra, rc, rn = O.kmeans(x, C, iters)
    assert np.array_equal(a, ra), int(np.sum(a != ra))
    assert np.array_equal(cnt, rn)
    n = np.maximum(rn, 1)[..., None].astype(np.float64)
    print(f"k-means C={C} iters={iters}: {ulps} near-tie choices; centroids max |gpu - oracle| "
          f"{float(np.abs(cent - rc).max()):.2e}")
    return a, cent, cnt


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("f32", [False, True])
def test_kmeans_and_layout(case, f32):
    grid, H, D, Cq, _, iters = case
    q, _, _ = _inputs(grid, H, D, 61)
    N = q.shape[1]
    ssa = SemanticSparseAttention(N, 1, H, D, Cq, Cq, iters=iters)
    qd = dev(q, torch.float32 if f32 else torch.bfloat16)
    a, _, _ = _check_kmeans(q, qd, Cq, iters)
    c = ssa.cluster(qd, Cq)
    assert np.array_equal(c.assign.cpu().numpy(), a)
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
    _check_kmeans(xr, xb, C, iters)


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
    # every query against attention under the GPU's own clusters and cluster selection
    # (the selection the forward consumed; its parity with the oracle's is checked above)
    ref = O.cluster_attention(q, k, v, res["qc"].assign.cpu().numpy(), res["kc"].assign.cpu().numpy(), Cq, Ck,
                              ssa.scale, crp_g, cci_g)
    e = np.abs(o.astype(np.float64) - ref).ravel()
    assert e.max() <= BF16_MAX_ABS and e.mean() <= BF16_MEAN_ABS, (e.max(), e.mean())


def test_semantic_full_480p_sampled():
    """The 480p shape with 128 query and 128 key clusters: the assignments of heads 0
    and 11 equal the oracle's k-means, their cluster masses (from the GPU's and the
    oracle's centroids) within an ulp, and outputs of sampled query tokens against
    attention under the oracle's selection."""
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
        # outputs against attention under the GPU's own clusters and selection of this head
        qa_g = res["qc"].assign.cpu().numpy()[:, h:h + 1]
        ka_g = res["kc"].assign.cpu().numpy()[:, h:h + 1]
        ref = O.cluster_attention(qh, kh, vh, qa_g, ka_g, ssa.Cq, ssa.Ck, ssa.scale, sub_rp, sub_ci, tokens=toks)
        e = np.abs(o[0, toks, h].astype(np.float64) - ref[0, 0])
        assert e.max() <= BF16_MAX_ABS and e.mean() <= BF16_MEAN_ABS, (h, e.max(), e.mean())


@pytest.mark.parametrize("NB,H,D,seed", [(37, 2, 128, 1), (40, 1, 128, 2), (23, 2, 64, 3)])
def test_varlen_forward_counted_blocks(NB, H, D, seed):
    """The forward over counted blocks on its own: key blocks with 0 .. 64 real keys
    (every prefix pattern of a 16-key tile occurs), runs of query blocks with the same
    row (as one query cluster gives) and neighbours with different rows, empty rows,
    repeated and out-of-range entries, and an odd block count (the last workgroup of
    a slice holds one query block). Each block is taken as one cluster, so the outputs
    are the oracle's attention under that cluster selection; lse against a float64
    library logsumexp over the allowed keys. Both calls: without lse (pre-scaled
    queries for D = 128) and with lse and float32 output."""
    rng = np.random.default_rng(seed)
    choices = np.array([0, 1, 3, 4, 5, 8, 12, 17, 24, 27, 28, 29, 31, 32, 33, 36, 40, 47, 59, 60, 63, 64])
    kcnt = np.where(rng.random((H, NB)) < 0.5, 64, rng.choice(choices, (H, NB))).astype(np.int32)
    qcnt = np.where(rng.random((H, NB)) < 0.6, 64, rng.choice(choices, (H, NB))).astype(np.int32)
    N = int(max(kcnt.sum(1).max(), qcnt.sum(1).max()))
    x = [rng.standard_normal((1, N, H, D)).astype(np.float32) for _ in range(3)]
    x[0] *= 1.5
    q, k, v = (torch.from_numpy(a).to(torch.bfloat16).float().numpy() for a in x)
    # slot maps: each block's first count slots hold distinct tokens; tokens left over
    # belong to an extra cluster NB that no row lists
    kslot = np.full((H, NB * 64), -1, np.int64)
    qslot = np.full((H, NB * 64), -1, np.int64)
    kassign = np.full((1, H, N), NB, np.int32)
    qassign = np.full((1, H, N), NB, np.int32)
    for h in range(H):
        for slot, cnt, assign in ((kslot, kcnt, kassign), (qslot, qcnt, qassign)):
            perm = rng.permutation(N)
            t = 0
            for b in range(NB):
                toks = perm[t:t + cnt[h, b]]
                slot[h, b * 64:b * 64 + len(toks)] = toks
                assign[0, h, toks] = b
                t += cnt[h, b]
    # rows: runs of 1..4 query blocks share one list; a few empty rows; some rows with
    # out-of-range entries (-2, NB + 3) and, for D = 128, a repeated entry
    rows = []
    for h in range(H):
        b = 0
        while b < NB:
            run = int(rng.integers(1, 5))
            lst = rng.permutation(NB)[: int(rng.integers(0, NB + 1))]
            if rng.random() < 0.1:
                lst = lst[:0]
            for _ in range(min(run, NB - b)):
                r = list(lst)
                if len(r) and rng.random() < 0.3:
                    # D = 64 walks rows in CSR order, where a repeat counts per listing
                    r = r + ([r[0]] if D == 128 else []) + [-2, NB + 3]
                    rng.shuffle(r)
                rows.append(np.array(r, np.int32))
                b += 1
    rp = np.zeros(H * NB + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.concatenate(rows).astype(np.int32) if rp[-1] else np.zeros(1, np.int32)
    # the oracle's cluster rows: the same lists plus an empty row for cluster NB
    orows = []
    for h in range(H):
        orows += rows[h * NB:(h + 1) * NB] + [np.zeros(0, np.int32)]
    orp = np.zeros(H * (NB + 1) + 1, np.int32)
    orp[1:] = np.cumsum([len(r) for r in orows])
    oci = np.concatenate(orows).astype(np.int32) if orp[-1] else np.zeros(0, np.int32)
    scale = 1.0 / np.sqrt(D)
    ref = O.cluster_attention(q, k, v, qassign, kassign, NB + 1, NB + 1, scale, orp, oci)

    def tiled(a, slot):
        out = np.zeros((1, H, NB * 64, D), np.float32)
        for h in range(H):
            real = slot[h] >= 0
            out[0, h, real] = a[0, slot[h][real], h]
        return out
    qt = dev(rows_to_qk(tiled(q, qslot), NB), torch.bfloat16)
    kt = dev(rows_to_qk(tiled(k, kslot), NB), torch.bfloat16)
    vt = dev(rows_to_vt(tiled(v, kslot), NB), torch.bfloat16)
    kc, rpd, cid = dev(kcnt, torch.int32), dev(rp, torch.int32), dev(ci, torch.int32)
    o1 = torch.empty((1, H, NB * 64, D), dtype=torch.bfloat16, device="cuda")
    o2, o32 = torch.empty_like(o1), torch.empty((1, H, NB * 64, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, H, NB * 64), dtype=torch.float32, device="cuda")
    fpsa.sparse_attn_fwd_varlen(qt, kt, vt, kc, rpd, cid, 1, H, D, NB, scale, o1)
    fpsa.sparse_attn_fwd_varlen(qt, kt, vt, kc, rpd, cid, 1, H, D, NB, scale, o2, lse=lse, o_f32=o32)
    o1, o2, o32, lse = (t.float().cpu().numpy() for t in (o1, o2, o32, lse))
    for h in range(H):
        real = qslot[h] >= 0
        want = ref[0, qslot[h][real], h]
        for got in (o1, o2, o32):
            e = np.abs(got[0, h, real].astype(np.float64) - want)
            assert e.max() <= BF16_MAX_ABS and e.mean() <= BF16_MEAN_ABS, (h, e.max(), e.mean())
        # lse: each real query against the allowed keys of its block's row
        for qb in range(NB):
            r = h * NB + qb
            kept = np.unique(ci[rp[r]:rp[r + 1]])
            kept = kept[(kept >= 0) & (kept < NB)]
            keys = np.concatenate([kslot[h, b * 64:b * 64 + kcnt[h, b]] for b in kept]) if len(kept) else []
            qs = qslot[h, qb * 64:qb * 64 + qcnt[h, qb]]
            if len(qs) == 0:
                continue
            got = lse[0, h, qb * 64:qb * 64 + len(qs)]
            if len(keys) == 0:
                assert np.all(np.isneginf(got)) and np.all(o1[0, h, qb * 64:(qb + 1) * 64] == 0)
                continue
            s = q[0, qs, h].astype(np.float64) @ k[0, keys, h].astype(np.float64).T * scale
            want_l = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
            assert np.abs(got - want_l).max() < 2e-3, (h, qb)
    # a repeated entry and out-of-range entries change nothing: the same rows cleaned
    if D == 128:
        clean = [np.unique(r[(r >= 0) & (r < NB)]) for r in rows]
        crp = np.zeros(H * NB + 1, np.int32)
        crp[1:] = np.cumsum([len(r) for r in clean])
        cci = np.concatenate(clean).astype(np.int32) if crp[-1] else np.zeros(1, np.int32)
        o3 = torch.empty((1, H, NB * 64, D), dtype=torch.bfloat16, device="cuda")
        fpsa.sparse_attn_fwd_varlen(qt, kt, vt, kc, dev(crp, torch.int32), dev(cci, torch.int32), 1, H, D, NB,
                                    scale, o3)
        assert np.array_equal(o3.float().cpu().numpy(), o1)
