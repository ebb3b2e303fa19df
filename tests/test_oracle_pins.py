"""Pins for the CPU oracle: each function is tied to something other than itself.

Sources of truth used here: closed forms worked out by hand, invariants of the
definitions, brute-force enumeration on tiny inputs, textbook softmax attention
computed by a library routine (torch's scaled_dot_product_attention in float64),
and the published OCP 8-bit floating-point (e4m3fn) code table.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_reorder_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


# --------------------------------------------------------------------------- geometry

def test_block_counts_of_the_workload_grids():
    # tiles per axis worked out by hand: ceil(21/4)=6, ceil(30/4)=8, 52/4=13 -> 624 ...
    assert O.num_blocks((4, 8, 8), (4, 4, 4)) == 4
    assert O.num_blocks((21, 30, 52), (4, 4, 4)) == 6 * 8 * 13
    assert O.num_blocks((21, 45, 80), (4, 4, 4)) == 6 * 12 * 20
    assert O.num_blocks((33, 45, 80), (4, 4, 4)) == 9 * 12 * 20
    assert O.num_blocks((1, 512, 512), (1, 8, 8)) == 64 * 64
    assert O.num_blocks((0, 4, 4), (4, 4, 4)) < 0


def test_token_slots_hand_values():
    blk, slot = O.token_blocks((21, 30, 52), (4, 4, 4))
    # token (t=5, h=7, w=50): tile (1, 1, 12) -> block (1*8 + 1)*13 + 12 = 129,
    # position inside the tile (1, 3, 2) -> (1*4 + 3)*4 + 2 = 30
    n = (5 * 30 + 7) * 52 + 50
    assert blk[n] == 129 and slot[n] == 129 * 64 + 30
    # first and last token
    assert blk[0] == 0 and slot[0] == 0
    n = 21 * 30 * 52 - 1             # (20, 29, 51): tile (5, 7, 12) -> 5*104+7*13+12 = 623
    assert blk[n] == 623 and slot[n] == 623 * 64 + (0 * 4 + 1) * 4 + 3
    # 2D image groups: token (h=9, w=17) -> group (1, 2) = 66, inside (1, 1) -> 9
    blk, slot = O.token_blocks((1, 512, 512), (1, 8, 8))
    n = 9 * 512 + 17
    assert blk[n] == 66 and slot[n] == 66 * 64 + 9


def test_token_slots_are_a_bijection_onto_real_slots():
    for grid in [(5, 6, 4), (21, 30, 52), (4, 8, 8), (7, 9, 13)]:
        blk, slot = O.token_blocks(grid, (4, 4, 4))
        assert len(np.unique(slot)) == len(slot)
        assert np.all(slot // 64 == blk)
        assert slot.min() >= 0 and slot.max() < 64 * O.num_blocks(grid, (4, 4, 4))


def test_block_sizes_ragged_hand_values():
    # grid 5x6x4 with 4^3 tiles: t-tiles hold 4 and 1 frames, h-tiles 4 and 2 rows
    sizes = O.block_sizes((5, 6, 4), (4, 4, 4))
    assert sizes.tolist() == [64, 32, 16, 8]
    # smallest blocks of the video workloads: 480p 1*2*4, 720p 1*1*4
    assert O.block_sizes((21, 30, 52), (4, 4, 4)).min() == 8
    assert O.block_sizes((21, 45, 80), (4, 4, 4)).min() == 4
    assert O.block_sizes((21, 30, 52), (4, 4, 4)).sum() == 21 * 30 * 52


# --------------------------------------------------------------------------- dense attention

def _rand_qkv(B, N, H, D, seed):
    g = np.random.default_rng(seed)
    return [g.standard_normal((B, N, H, D)).astype(np.float32) for _ in range(3)]


def _torch_sdpa(q, k, v, scale):
    # library routine, float64, [B, H, N, D] layout
    t = lambda a: torch.from_numpy(a.astype(np.float64)).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def test_dense_attention_matches_library_softmax_attention():
    q, k, v = _rand_qkv(2, 70, 3, 16, 1)
    ref = _torch_sdpa(q, k, v, 0.25)
    got = O.dense_attention(q, k, v, 0.25)
    assert np.abs(got - ref).max() < 1e-12


def test_dense_attention_zero_query_is_mean_of_values():
    q, k, v = _rand_qkv(1, 50, 2, 8, 2)
    q[:] = 0
    got = O.dense_attention(q, k, v, 0.3)
    assert np.abs(got - v.astype(np.float64).mean(axis=1, keepdims=True)).max() < 1e-12


# --------------------------------------------------------------------------- block masses

def test_mass_rows_sum_to_one_on_a_ragged_grid():
    grid, tile = (5, 6, 7), (4, 4, 4)
    N = 5 * 6 * 7
    q, k, _ = _rand_qkv(1, N, 2, 16, 3)
    M = O.block_mass(q * 2, k * 2, grid, tile, 0.25)
    assert np.abs(M.sum(-1) - 1).max() < 1e-12
    assert M.min() >= 0


def test_mass_zero_query_is_key_count_share():
    grid, tile = (5, 6, 4), (4, 4, 4)
    q, k, _ = _rand_qkv(1, 120, 1, 8, 4)
    q[:] = 0
    M = O.block_mass(q, k, grid, tile, 1.0)
    want = np.array([64, 32, 16, 8]) / 120.0
    assert np.abs(M[0, 0] - want).max() < 1e-13


def test_mass_single_block_is_one():
    q, k, _ = _rand_qkv(1, 64, 2, 8, 5)
    M = O.block_mass(q, k, (4, 4, 4), (4, 4, 4), 0.5)
    assert M.shape == (1, 2, 1, 1) and np.abs(M - 1).max() < 1e-13


def test_mass_closed_form_with_blockwise_constant_scores():
    # every query = alpha*e0, every key of block b = beta_b*e0, so the score of any
    # query against block b is scale*alpha*beta_b and the mass of b is
    # c(b) e^{s_b} / sum_b' c(b') e^{s_b'} for every query block.
    grid, tile = (5, 6, 4), (4, 4, 4)
    sizes = np.array([64, 32, 16, 8], dtype=np.float64)
    blk, _ = O.token_blocks(grid, tile)
    beta = np.array([0.5, -1.0, 2.0, 1.25])
    q = np.zeros((1, 120, 1, 8), np.float32); q[..., 0] = 1.5
    k = np.zeros((1, 120, 1, 8), np.float32); k[0, :, 0, 0] = beta[blk]
    scale = 0.75
    s = scale * 1.5 * beta
    want = sizes * np.exp(s) / np.sum(sizes * np.exp(s))
    M = O.block_mass(q, k, grid, tile, scale)
    for qb in range(4):
        assert np.abs(M[0, 0, qb] - want).max() < 1e-13


def test_mass_subset_rows_equal_full_rows():
    grid, tile = (4, 8, 12), (4, 4, 4)
    q, k, _ = _rand_qkv(1, 4 * 8 * 12, 2, 16, 6)
    full = O.block_mass(q, k, grid, tile, 0.3)
    part = O.block_mass(q, k, grid, tile, 0.3, qblocks=[5, 0, 3])
    assert np.array_equal(part, full[:, :, [5, 0, 3]])


def test_mass_follows_swapped_key_blocks():
    # swapping the keys of two equal-sized blocks swaps their mass columns
    grid, tile = (4, 8, 8), (4, 4, 4)
    q, k, _ = _rand_qkv(1, 256, 1, 16, 7)
    blk, _ = O.token_blocks(grid, tile)
    a, b = np.where(blk == 1)[0], np.where(blk == 2)[0]
    k2 = k.copy(); k2[:, a], k2[:, b] = k[:, b], k[:, a]
    M, M2 = O.block_mass(q, k, grid, tile, 0.3), O.block_mass(q, k2, grid, tile, 0.3)
    assert np.abs(M2[..., [0, 2, 1, 3]] - M).max() < 1e-14


# --------------------------------------------------------------------------- selection

def test_mass_key_exact_values():
    assert O.mass_key(0.5) == 2 ** 39
    assert O.mass_key(1.0) == 2 ** 40
    assert O.mass_key(3.0) == 2 ** 40
    assert O.mass_key(2.0 ** -40) == 1
    assert O.mass_key(2.0 ** -41) == 0
    assert O.mass_key(0.0) == 0 and O.mass_key(-0.25) == 0 and O.mass_key(float("nan")) == 0
    m = float(np.float32(0.1))
    assert O.mass_key(m) == math.floor(m * 2 ** 40)


def _csr_rows(rp, ci):
    return [ci[rp[r]:rp[r + 1]].tolist() for r in range(len(rp) - 1)]


def test_selection_hand_examples():
    row = np.array([[1 / 2, 1 / 4, 1 / 8, 1 / 16, 1 / 32, 1 / 32]], np.float32)
    assert _csr_rows(*O.select_blocks(row, 99, 100)) == [[0, 1, 2, 3, 4, 5]]
    assert _csr_rows(*O.select_blocks(row, 1, 2)) == [[0]]          # exactly half: >= holds
    assert _csr_rows(*O.select_blocks(row, 3, 4)) == [[0, 1]]
    assert _csr_rows(*O.select_blocks(row, 15, 16)) == [[0, 1, 2, 3]]
    # ties go to the lower block index
    row = np.full((1, 4), 0.25, np.float32)
    assert _csr_rows(*O.select_blocks(row, 1, 2)) == [[0, 1]]
    row = np.array([[0.1, 0.3, 0.3, 0.3]], np.float32)
    assert _csr_rows(*O.select_blocks(row, 1, 2)) == [[1, 2]]
    # all-zero row keeps nothing; so does a zero threshold
    assert _csr_rows(*O.select_blocks(np.zeros((1, 5), np.float32))) == [[]]
    assert _csr_rows(*O.select_blocks(np.ones((1, 3), np.float32) / 3, 0, 100)) == [[]]
    # kept indices come out ascending even when the ranking is not
    row = np.array([[0.05, 0.6, 0.05, 0.3]], np.float32)
    assert _csr_rows(*O.select_blocks(row, 9, 10)) == [[1, 3]]


def _brute_force_select(row, num, den):
    keys = [math.floor(float(x) * 2 ** 40) if x > 0 else 0 for x in row]
    keys = [min(kk, 2 ** 40) for kk in keys]
    S = sum(keys)
    nb = len(row)
    for size in range(0, nb + 1):
        best = None
        for sub in itertools.combinations(range(nb), size):
            c = sum(keys[i] for i in sub)
            if den * c >= num * S:
                cand = (-c, list(sub))
                if best is None or cand < best:
                    best = cand
        if best is not None:
            return best[1]
    raise AssertionError("unreachable")


@pytest.mark.parametrize("nb,num,den", [(4, 99, 100), (8, 99, 100), (10, 9, 10), (12, 99, 100), (9, 1, 2)])
def test_selection_equals_brute_force(nb, num, den):
    rows = synth.random_mass_rows(24 if nb <= 10 else 6, nb, seed=nb * 7 + num, tie_frac=0.3, zero_frac=0.1)
    # add rows with heavy exact ties
    rows = np.concatenate([rows, np.full((1, nb), 1.0 / nb, np.float32)])
    got = _csr_rows(*O.select_blocks(rows, num, den))
    for r in range(rows.shape[0]):
        assert got[r] == _brute_force_select(rows[r], num, den), r


def test_selection_is_minimal_and_rank_consistent():
    rows = synth.random_mass_rows(300, 97, seed=11)
    rp, ci = O.select_blocks(rows)
    for r in range(rows.shape[0]):
        keys = np.array([O.mass_key(x) for x in rows[r]], dtype=object)
        kept = ci[rp[r]:rp[r + 1]]
        S, C = int(keys.sum()), int(keys[kept].sum())
        assert 100 * C >= 99 * S
        if len(kept):
            weakest = min(kept, key=lambda i: (keys[i], -i))
            assert 100 * (C - int(keys[weakest])) < 99 * S
        dropped = np.setdiff1d(np.arange(rows.shape[1]), kept)
        for d in dropped:
            for kk in kept:
                assert (keys[kk] > keys[d]) or (keys[kk] == keys[d] and kk < d)


def test_cut_margin_of_dyadic_row():
    # masses 0.5, 0.3, 0.2 at p = 0.75: keep 2, c = 0.8, prev = 0.5, gap 0.1
    m = O.cut_margin(np.array([[0.5, 0.3, 0.2]]), 0.75)
    assert abs(m[0] - 0.05) < 1e-15


# --------------------------------------------------------------------------- masked attention

def test_all_blocks_mask_equals_dense_attention():
    grid, tile = (5, 6, 7), (4, 4, 4)
    N, nb = 210, O.num_blocks(grid, tile)
    q, k, v = _rand_qkv(1, N, 2, 16, 8)
    rp = np.arange(0, 2 * nb * nb + 1, nb, dtype=np.int32)
    ci = np.tile(np.arange(nb, dtype=np.int32), 2 * nb)
    out, tok = O.masked_attention(q, k, v, grid, tile, 0.25, rp, ci)
    dense = _torch_sdpa(q, k, v, 0.25)
    for h in range(2):
        for qb in range(nb):
            t = tok[0, h, qb]
            t = t[t >= 0]
            assert np.abs(out[0, h, qb, :len(t)] - dense[0, t, h]).max() < 1e-12


def test_single_kept_block_is_attention_within_that_block():
    grid, tile = (4, 8, 8), (4, 4, 4)
    q, k, v = _rand_qkv(1, 256, 1, 16, 9)
    blk, _ = O.token_blocks(grid, tile)
    rp = np.array([0, 1, 2, 2, 3], np.int32)           # qb0->{2}, qb1->{0}, qb2->{}, qb3->{3}
    ci = np.array([2, 0, 3], np.int32)
    out, tok = O.masked_attention(q, k, v, grid, tile, 0.4, rp, ci)
    for qb, kb in [(0, 2), (1, 0), (3, 3)]:
        qs, ks = np.where(blk == qb)[0], np.where(blk == kb)[0]
        ref = _torch_sdpa(q[:, qs], k[:, ks], v[:, ks], 0.4)
        assert np.array_equal(tok[0, 0, qb], qs)
        assert np.abs(out[0, 0, qb] - ref[0, :, 0]).max() < 1e-12
    assert np.all(out[0, 0, 2] == 0)                   # empty row: zero output


def test_out_of_range_blocks_contribute_nothing():
    # the ABI defines CSR entries outside [0, nb) as contributing nothing: with such
    # entries mixed in (negative, nb, far past nb) each row equals library attention
    # over the keys of its in-range blocks, and a row of only bad entries is zero
    grid, tile = (4, 8, 8), (4, 4, 4)
    q, k, v = _rand_qkv(1, 256, 1, 16, 29)
    blk, _ = O.token_blocks(grid, tile)
    rp = np.array([0, 4, 6, 8, 9], np.int32)
    ci = np.array([2, -1, 3, 4, 0, 1 << 30, -7, 99, 3], np.int32)
    out, tok = O.masked_attention(q, k, v, grid, tile, 0.4, rp, ci)
    for qb, kbs in [(0, [2, 3]), (1, [0]), (3, [3])]:
        qs, ks = np.where(blk == qb)[0], np.where(np.isin(blk, kbs))[0]
        ref = _torch_sdpa(q[:, qs], k[:, ks], v[:, ks], 0.4)
        assert np.abs(out[0, 0, qb] - ref[0, :, 0]).max() < 1e-12
    assert np.all(out[0, 0, 2] == 0)


def test_masked_attention_constant_values_give_constant_output():
    grid, tile = (5, 6, 7), (4, 4, 4)
    q, k, v = _rand_qkv(1, 210, 1, 8, 10)
    v[:] = 0.375
    nb = O.num_blocks(grid, tile)
    rows = synth.random_mass_rows(nb, nb, seed=3)
    rp, ci = O.select_blocks(rows, 1, 2)
    out, tok = O.masked_attention(q, k, v, grid, tile, 0.3, rp, ci)
    for qb in range(nb):
        n = int((tok[0, 0, qb] >= 0).sum())
        expect = 0.375 if rp[qb + 1] > rp[qb] else 0.0
        assert np.abs(out[0, 0, qb, :n] - expect).max() < 1e-14


# --------------------------------------------------------------------------- fp8 e4m3

def test_e4m3_code_table():
    # OCP 8-bit floating point spec, E4M3 (bias 7, no infinities, S.1111.111 = NaN)
    assert O.e4m3_decode(0x00) == 0.0 and math.copysign(1, O.e4m3_decode(0x80)) < 0
    assert O.e4m3_decode(0x01) == 2.0 ** -9                   # smallest subnormal
    assert O.e4m3_decode(0x07) == 7 * 2.0 ** -9               # largest subnormal
    assert O.e4m3_decode(0x08) == 2.0 ** -6                   # smallest normal
    assert O.e4m3_decode(0x38) == 1.0
    assert O.e4m3_decode(0x39) == 1.125
    assert O.e4m3_decode(0x40) == 2.0 and O.e4m3_decode(0x44) == 3.0
    assert O.e4m3_decode(0x7E) == 448.0 and O.e4m3_decode(0xFE) == -448.0
    assert O.e4m3_decode(0x78) == 256.0
    assert math.isnan(O.e4m3_decode(0x7F)) and math.isnan(O.e4m3_decode(0xFF))
    mags = [O.e4m3_decode(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(mags, mags[1:]))
    assert len([c for c in range(256) if math.isnan(O.e4m3_decode(c))]) == 2


def test_e4m3_encode_roundtrip_rne_and_saturation():
    for c in list(range(0x7F)) + list(range(0x81, 0xFF)):
        assert O.e4m3_encode(O.e4m3_decode(c)) == c
    assert O.e4m3_encode(1.0625) == 0x38      # midpoint 1 / 1.125 -> even code
    assert O.e4m3_encode(1.1875) == 0x3A      # midpoint 1.125 / 1.25 -> even code
    assert O.e4m3_encode(1.0626) == 0x39
    assert O.e4m3_encode(2.0 ** -10) == 0x00  # half the smallest subnormal -> even (zero)
    assert O.e4m3_encode(3 * 2.0 ** -10) == 0x02
    assert O.e4m3_encode(449.0) == 0x7E and O.e4m3_encode(464.0) == 0x7E
    assert O.e4m3_encode(1e9) == 0x7E and O.e4m3_encode(-1e9) == 0xFE
    assert O.e4m3_encode(-3.0) == 0xC4


def test_fp8_tile_quantize_scales_and_error():
    grid, tile = (5, 6, 4), (4, 4, 4)
    x = _rand_qkv(1, 120, 2, 16, 12)[0]
    blk, _ = O.token_blocks(grid, tile)
    x[0, blk == 2, 1, :] = 0.0                               # an all-zero tile
    xhat, sc = O.fp8_tile_quantize(x, grid, tile)
    for h in range(2):
        for b in range(4):
            sel = x[0, blk == b, h, :]
            if np.all(sel == 0):
                assert sc[0, h, b] == 1.0
                continue
            amax = np.float32(np.abs(sel).max())
            assert sc[0, h, b] == np.float32(amax / np.float32(448.0))
            xs = xhat[0, blk == b, h, :]
            # the largest element lands on 448 * scale; e4m3 relative step <= 2^-3 for normals
            assert np.isclose(np.abs(xs).max(), 448.0 * sc[0, h, b], rtol=1e-6)
            big = np.abs(sel) > 2.0 ** -6 * sc[0, h, b]
            assert np.all(np.abs(xs[big] - sel[big]) <= 2.0 ** -4 * np.abs(sel[big]) * 1.0001)


# --------------------------------------------------------------------------- structured mask

def test_structured_mask_counts_by_hand():
    # interior group: its row (64) + its column (64) - itself + 4 diagonal neighbours = 131;
    # border groups lose 2 diagonals (129), corners lose 3 (128)
    rp, ci = O.structured_mask(64, 64)
    counts = np.diff(rp)
    assert len(ci) == 4 * 128 + 4 * 62 * 129 + 62 * 62 * 131 == 536068
    vals, freq = np.unique(counts, return_counts=True)
    assert dict(zip(vals.tolist(), freq.tolist())) == {128: 4, 129: 248, 131: 3844}


def test_structured_mask_small_grid_by_enumeration():
    rp, ci = O.structured_mask(3, 4)
    rows = _csr_rows(rp, ci)
    # group (1, 1) = id 5: everything in row 1, column 1, and the 3x3 around it
    assert rows[5] == [0, 1, 2, 4, 5, 6, 7, 8, 9, 10]
    # corner (0, 0): row 0, column 0, and (1, 1)
    assert rows[0] == [0, 1, 2, 3, 4, 5, 8]
    rp2, ci2 = O.structured_mask(3, 4, copies=2)
    assert _csr_rows(rp2, ci2) == rows + rows


def test_fp8_tile_codes_decode_to_quantized_values():
    grid, tile = (5, 6, 4), (4, 4, 4)
    x = _rand_qkv(1, 120, 2, 16, 13)[0] * 7
    codes, sc = O.fp8_tile_codes(x, grid, tile)
    xhat, sc2 = O.fp8_tile_quantize(x, grid, tile)
    blk, _ = O.token_blocks(grid, tile)
    assert np.array_equal(sc, sc2)
    dec = np.vectorize(O.e4m3_decode)(codes)
    s = sc[0][:, blk].T[None, :, :, None]                 # [1, N, H, 1]
    assert np.array_equal((dec * s).astype(np.float32), xhat)


# --------------------------------------------------------------------------- retained-mass monitor

def test_retained_mass_hand_values_and_degenerate_rows():
    m = np.array([[0.5, 0.25, 0.125, 0.125],
                  [0.1, 0.2, 0.3, 0.4],
                  [1.0, 0.0, 0.0, 0.0]], np.float32)
    rp = np.array([0, 2, 2, 6], np.int32)
    # row 0 keeps {0, 2}; row 1 keeps nothing; row 2 lists 3 twice, -1 and 4 (out of range)
    ci = np.array([2, 0, 3, 3, -1, 4], np.int32)
    out = O.retained_mass(m, rp, ci)
    assert out.tolist() == [0.625, 0.0, 0.0]
    # leading shapes flatten to rows
    out2 = O.retained_mass(m.reshape(1, 3, 4), rp, ci)
    assert out2.tolist() == out.tolist()


def test_retained_mass_of_full_rows_is_one_and_of_selection_clears_threshold():
    grid, tile = (5, 6, 7), (4, 4, 4)
    nb = O.num_blocks(grid, tile)
    q, k, _ = _rand_qkv(1, 210, 2, 16, 21)
    mass = O.block_mass(q, k, grid, tile, 0.25).reshape(-1, nb)
    full_rp = np.arange(0, mass.shape[0] * nb + 1, nb, dtype=np.int32)
    full_ci = np.tile(np.arange(nb, dtype=np.int32), mass.shape[0])
    assert np.abs(O.retained_mass(mass, full_rp, full_ci) - 1.0).max() < 1e-6
    # the 99 % selection of the same step keeps at least 99 % of each row's
    # (float32-stored) mass, up to the selection's 2^-40 key quantum per block
    rp, ci = O.select_blocks(mass)
    kept = O.retained_mass(mass, rp, ci)
    tot = mass.astype(np.float64).sum(axis=1)
    assert np.all(kept >= 0.99 * tot - nb * 2.0 ** -40)
    # and dropping its smallest kept block falls below
    for r in range(mass.shape[0]):
        row = ci[rp[r]:rp[r + 1]]
        w = min(row, key=lambda i: (mass[r, i], -i))
        assert kept[r] - mass[r, w] < 0.99 * tot[r] + nb * 2.0 ** -40


# --------------------------------------------------------------------------- fixed patterns

def test_pattern_mask_counts_by_closed_form():
    nb = 37
    # diagonal band w: row qb keeps min(qb+w, nb-1) - max(qb-w, 0) + 1 blocks;
    # in total nb(2w+1) - w(w+1)
    for w in (0, 1, 3):
        rp, ci = O.pattern_mask(nb, 1, 1, [(w, 0, 0, 0)])
        assert len(ci) == nb * (2 * w + 1) - w * (w + 1)
        assert np.diff(rp).tolist() == [min(q + w, nb - 1) - max(q - w, 0) + 1 for q in range(nb)]
    # vertical stripe s alone: every row keeps exactly blocks 0..s-1
    rp, ci = O.pattern_mask(nb, 1, 1, [(-1, 0, 5, 0)])
    assert _csr_rows(rp, ci) == [list(range(5))] * nb
    # dense: all nb
    rp, ci = O.pattern_mask(nb, 1, 1, [(-1, 0, 0, 1)])
    assert _csr_rows(rp, ci) == [list(range(nb))] * nb
    # nothing enabled: every row empty
    rp, ci = O.pattern_mask(nb, 1, 1, [(-1, 0, 0, 0)])
    assert len(ci) == 0 and np.all(rp == 0)


def test_pattern_mask_multi_diagonal_is_residue_classes():
    # band 0, period p dividing nb: row qb keeps exactly the blocks congruent to qb mod p
    nb, p = 48, 12
    rows = _csr_rows(*O.pattern_mask(nb, 1, 1, [(0, p, 0, 0)]))
    for q in range(nb):
        assert rows[q] == [k for k in range(q % p, nb, p)]
    # band w < p/2: 2w+1 residues around qb, so (2w+1) nb/p blocks per row
    rows = _csr_rows(*O.pattern_mask(nb, 1, 1, [(2, p, 0, 0)]))
    for q in range(nb):
        res = {(q + d) % p for d in range(-2, 3)}
        assert rows[q] == [k for k in range(nb) if k % p in res]
        assert len(rows[q]) == 5 * nb // p


def test_pattern_mask_heads_batches_and_union():
    nb = 20
    parts = [(1, 0, 0, 0), (-1, 0, 3, 0), (0, 5, 0, 0)]
    union = (1, 5, 3, 0)
    single = [_csr_rows(*O.pattern_mask(nb, 1, 1, [p])) for p in parts]
    both = _csr_rows(*O.pattern_mask(nb, 1, 1, [union]))
    for q in range(nb):
        assert both[q] == sorted(set(single[0][q]) | set(single[1][q]) | set(
            k for k in range(nb) if min((k - q) % 5, (q - k) % 5) <= 1))
    # rows are laid out (b, h, qb) with each head's own pattern
    rp, ci = O.pattern_mask(nb, 2, 3, parts)
    rows = _csr_rows(rp, ci)
    for b in range(2):
        for h in range(3):
            assert rows[(b * 3 + h) * nb:(b * 3 + h + 1) * nb] == single[h]
    # band patterns are symmetric: kb in row qb iff qb in row kb
    sym = _csr_rows(*O.pattern_mask(nb, 1, 1, [(2, 7, 0, 0)]))
    for q in range(nb):
        for k in sym[q]:
            assert q in sym[k]


# --------------------------------------------------------------------------- backward

def _token_mask(grid, tile, H, rp, ci):
    """[H, N, N] bool: query i may attend key j (key block kept by i's block row)."""
    blk, _ = O.token_blocks(grid, tile)
    nb = O.num_blocks(grid, tile)
    keep = np.zeros((H, nb, nb), bool)
    for h in range(H):
        for qb in range(nb):
            keep[h, qb, ci[rp[h * nb + qb]:rp[h * nb + qb + 1]]] = True
    return keep[:, blk][:, :, blk]


def _torch_grads(q, k, v, g, scale, mask):
    # library autograd through masked softmax attention, float64, [B, H, N, D]
    t = lambda a: torch.from_numpy(a.astype(np.float64)).permute(0, 2, 1, 3).clone().requires_grad_(True)
    tq, tk, tv = t(q), t(k), t(v)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask)[None],
                                                         scale=scale)
    o.backward(torch.from_numpy(g.astype(np.float64)).permute(0, 2, 1, 3))
    back = lambda x: x.grad.permute(0, 2, 1, 3).numpy()
    return back(tq), back(tk), back(tv)


def test_backward_matches_library_autograd():
    grid, tile, H, D = (5, 6, 7), (4, 4, 4), 2, 16
    nb = O.num_blocks(grid, tile)
    q, k, v = _rand_qkv(1, 210, H, D, 41)
    g = _rand_qkv(1, 210, H, D, 42)[0]
    rows = synth.random_mass_rows(H * nb, nb, seed=5)
    rp, ci = O.select_blocks(rows, 1, 2)
    dq, dk, dv = O.masked_attention_bwd(q, k, v, g, grid, tile, 0.3, rp, ci)
    rq, rk, rv = _torch_grads(q, k, v, g, 0.3, _token_mask(grid, tile, H, rp, ci))
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.abs(a - b).max() < 1e-11


def test_backward_matches_finite_differences_of_the_forward_oracle():
    grid, tile, H, D = (4, 8, 8), (4, 4, 4), 1, 8
    nb = O.num_blocks(grid, tile)
    q, k, v = _rand_qkv(1, 256, H, D, 43)
    g = _rand_qkv(1, 256, H, D, 44)[0]
    rp = np.array([0, 2, 3, 3, 5], np.int32)            # block 2 keeps nothing
    ci = np.array([0, 3, 1, 2, 3], np.int32)
    dq, dk, dv = O.masked_attention_bwd(q, k, v, g, grid, tile, 0.5, rp, ci)
    blk, _ = O.token_blocks(grid, tile)

    def loss(q_, k_, v_):
        out, tok = O.masked_attention(q_, k_, v_, grid, tile, 0.5, rp, ci)
        tot = 0.0
        for qb in range(nb):
            t = tok[0, 0, qb][tok[0, 0, qb] >= 0]
            tot += float(np.sum(out[0, 0, qb, :len(t)] * g[0, t, 0].astype(np.float64)))
        return tot

    rng = np.random.default_rng(0)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(4):
            n, d = int(rng.integers(0, 256)), int(rng.integers(0, D))
            plus, minus = [x.copy() for x in (q, k, v)], [x.copy() for x in (q, k, v)]
            plus[which][0, n, 0, d] += np.float32(1e-3)
            minus[which][0, n, 0, d] -= np.float32(1e-3)
            step = float(plus[which][0, n, 0, d]) - float(minus[which][0, n, 0, d])
            fd = (loss(*plus) - loss(*minus)) / step
            assert abs(fd - grad[0, n, 0, d]) < 1e-5 * max(1.0, abs(fd)), (which, n, d, fd, grad[0, n, 0, d])
    # queries of the block with no kept key get no gradient; nothing flows to its keys from them
    assert np.all(dq[0, blk == 2] == 0)


def test_backward_sums_over_keys():
    # sum_j ds_ij = 0 for every query, so the key gradients sum to zero; the value
    # gradients sum to the upstream gradients of the queries that attend anything
    grid, tile, H, D = (9, 10, 13), (4, 4, 4), 2, 16
    nb = O.num_blocks(grid, tile)
    N = 9 * 10 * 13
    q, k, v = _rand_qkv(1, N, H, D, 45)
    g = _rand_qkv(1, N, H, D, 46)[0]
    rows = synth.random_mass_rows(H * nb, nb, seed=6)
    rows[3] = 0.0                                       # one empty row
    rp, ci = O.select_blocks(rows, 9, 10)
    dq, dk, dv = O.masked_attention_bwd(q, k, v, g, grid, tile, 0.25, rp, ci)
    blk, _ = O.token_blocks(grid, tile)
    assert np.abs(dk.sum(axis=1)).max() < 1e-10
    for h in range(H):
        live = np.diff(rp)[h * nb + blk] > 0
        want = g[0, live, h].astype(np.float64).sum(axis=0)
        assert np.abs(dv[0, :, h].sum(axis=0) - want).max() < 1e-9
    # the sampled query-gradient routine gives the same rows
    sel = [0, 3, nb - 1]
    dqs, tok = O.masked_attention_bwd_dq(q, k, v, g, grid, tile, 0.25, rp, ci, sel)
    for h in range(H):
        for r in range(len(sel)):
            t = tok[0, h, r][tok[0, h, r] >= 0]
            assert np.array_equal(dqs[0, h, r, :len(t)], dq[0, t, h])


def test_csr_transpose_hand_example_and_round_trip():
    # 1 batch, 2 heads, 3 blocks
    rp = np.array([0, 2, 3, 3, 4, 7, 8], np.int32)
    ci = np.array([0, 2, 2, 1, 0, 1, 2, 1], np.int32)
    cp, ri = O.csr_transpose(rp, ci, 1, 2, 3)
    assert _csr_rows(cp, ri) == [[0], [], [0, 1], [1], [0, 1, 2], [1]]
    rows = synth.random_mass_rows(3 * 40, 40, seed=8)
    rp, ci = O.select_blocks(rows, 1, 2)
    cp, ri = O.csr_transpose(rp, ci, 1, 3, 40)
    rp2, ci2 = O.csr_transpose(cp, ri, 1, 3, 40)
    assert np.array_equal(rp2, rp) and np.array_equal(ci2, ci)
    # out-of-range entries dropped, repeats collapse
    cp, ri = O.csr_transpose(np.array([0, 4, 4], np.int32), np.array([1, 1, -1, 5], np.int32), 1, 1, 2)
    assert _csr_rows(cp, ri) == [[], [0]]


def test_backward_term_magnitudes():
    # triangle inequality everywhere; equality for dv when every upstream gradient is
    # non-negative (all its terms p_ij dout_i share a sign)
    grid, tile, H, D = (5, 6, 7), (4, 4, 4), 2, 16
    nb = O.num_blocks(grid, tile)
    q, k, v = _rand_qkv(1, 210, H, D, 47)
    g = np.abs(_rand_qkv(1, 210, H, D, 48)[0])
    rp, ci = O.select_blocks(synth.random_mass_rows(H * nb, nb, seed=7), 9, 10)
    dq, dk, dv, mq, mk, mv = O.masked_attention_bwd(q, k, v, g, grid, tile, 0.25, rp, ci, magnitudes=True)
    dq2, dk2, dv2 = O.masked_attention_bwd(q, k, v, g, grid, tile, 0.25, rp, ci)
    assert np.array_equal(dq, dq2) and np.array_equal(dk, dk2) and np.array_equal(dv, dv2)
    for a, m in ((dq, mq), (dk, mk), (dv, mv)):
        assert np.all(np.abs(a) <= m * (1 + 1e-12) + 1e-300)
    assert np.abs(dv - mv).max() < 1e-12
    sel = [1, nb - 1]
    dqs, mqs, tok = O.masked_attention_bwd_dq(q, k, v, g, grid, tile, 0.25, rp, ci, sel, magnitudes=True)
    for h in range(H):
        for r in range(len(sel)):
            t = tok[0, h, r][tok[0, h, r] >= 0]
            assert np.array_equal(mqs[0, h, r, :len(t)], mq[0, t, h])


# --------------------------------------------------------------------------- k-means permutation

def test_kmeans_recovers_separated_blobs():
    # C blobs of m consecutive tokens around far-apart centres: the strided start puts
    # one centroid in each blob, so one step finds the blobs and their means
    C, m, D, H = 6, 20, 8, 2
    rng = np.random.default_rng(3)
    centres = rng.standard_normal((H, C, D)) * 100
    x = np.zeros((1, C * m, H, D), np.float32)
    for h in range(H):
        for c in range(C):
            x[0, c * m:(c + 1) * m, h] = centres[h, c] + 0.01 * rng.standard_normal((m, D))
    a, cent, cnt = O.kmeans(x, C, 1)
    assert np.array_equal(a[0], np.tile(np.repeat(np.arange(C), m), (H, 1)))
    assert np.all(cnt == m)
    for h in range(H):
        for c in range(C):
            mean = x[0, c * m:(c + 1) * m, h].astype(np.float64).mean(axis=0)
            assert np.abs(cent[0, h, c] - mean).max() < 1e-9


def test_kmeans_hand_example_ties_and_empty_cluster():
    # start: centroid 0 = token 0, centroid 1 = token 2, both equal to a: every token
    # is equally far from both and goes to cluster 0; cluster 1 stays empty and keeps
    # its starting point
    a_, b_, c_ = [1.0, 2.0], [3.0, -1.0], [0.0, 5.0]
    x = np.array([[a_, b_, a_, c_]], np.float32)[:, :, None, :]
    asg, cent, cnt = O.kmeans(x, 2, 1)
    assert asg[0, 0].tolist() == [0, 0, 0, 0] and cnt[0, 0].tolist() == [4, 0]
    assert np.allclose(cent[0, 0, 0], np.mean([a_, b_, a_, c_], axis=0), atol=1e-15)
    assert cent[0, 0, 1].tolist() == a_
    # second step by hand: centroids (1.25, 2) and (1, 2); a is nearer the second
    # (0 < 1/16), b the first (12.0625 < 13), c the second (10 < 10.5625)
    asg, cent, cnt = O.kmeans(x, 2, 2)
    assert asg[0, 0].tolist() == [1, 0, 1, 1] and cnt[0, 0].tolist() == [1, 3]
    assert cent[0, 0, 0].tolist() == b_
    assert np.allclose(cent[0, 0, 1], [2.0 / 3.0, 3.0], atol=1e-15)


def test_kmeans_lloyd_properties():
    x = _rand_qkv(1, 300, 2, 6, 9)[0]
    objective = []
    for iters in range(1, 7):
        a, cent, cnt = O.kmeans(x, 7, iters)
        for h in range(2):
            for c in range(7):
                mem = np.where(a[0, h] == c)[0]
                assert cnt[0, h, c] == len(mem)
                if len(mem):
                    assert np.abs(cent[0, h, c] - x[0, mem, h].astype(np.float64).mean(axis=0)).max() < 1e-12
        objective.append(sum(np.sum((x[0, :, h].astype(np.float64) - cent[0, h][a[0, h]]) ** 2) for h in range(2)))
    # Lloyd never increases the within-cluster sum of squares
    assert all(objective[i + 1] <= objective[i] + 1e-9 for i in range(len(objective) - 1))
    # after many steps the assignment is a fixed point: every token's nearest centroid
    a, cent, _ = O.kmeans(x, 7, 60)
    for h in range(2):
        d = ((x[0, :, h, None, :].astype(np.float64) - cent[0, h][None]) ** 2).sum(-1)
        assert np.array_equal(np.argmin(d, axis=1), a[0, h])


def test_kmeans_assignment_is_the_exact_nearest_centroid():
    # every assignment step against exact rational arithmetic: the squared distance
    # sum_d (x_d - c_d)^2 to the centroids the step starts from (the starting tokens,
    # or the centroids the oracle returns after one step fewer), least value, ties to
    # the lower cluster; the oracle sums the float64 squares of the differences
    _exact_nearest_steps(_rand_qkv(1, 40, 2, 8, 11)[0], 5, 4)
    _exact_nearest_steps(_rand_qkv(1, 150, 1, 16, 12)[0] * np.float32(0.25), 9, 3)


def _exact_nearest_steps(x, C, steps):
    from fractions import Fraction as Fr
    N = x.shape[1]
    for iters in range(1, steps + 1):
        asg, _, _ = O.kmeans(x, C, iters)
        for h in range(x.shape[2]):
            if iters == 1:
                cent = [x[0, c * N // C, h].astype(np.float64) for c in range(C)]
            else:
                cent = O.kmeans(x, C, iters - 1)[1][0, h]
            for n in range(N):
                xn = [Fr(float(v)) for v in x[0, n, h]]
                dist = [sum((a - Fr(float(cv))) ** 2 for a, cv in zip(xn, cent[c])) for c in range(C)]
                assert asg[0, h, n] == min(range(C), key=lambda c: (dist[c], c))


def test_kmeans_assign_step_excess_and_tolerance():
    # the checking form of one assignment step: against exact rational distances, the
    # excess of another choice is its distance less the nearest one's (up to float64
    # rounding of the two sums), zero when the choices agree, and the tolerance is a
    # small positive bound that a clearly farther centroid exceeds
    from fractions import Fraction as Fr
    x = _rand_qkv(1, 60, 2, 8, 21)[0]
    cent = O.kmeans(x, 6, 2)[1]
    a = O.kmeans_assign(x, cent)
    assert np.array_equal(a, O.kmeans(x, 6, 3)[0])           # the step the clustering takes
    _, ex0, tol0 = O.kmeans_assign(x, cent, other=a)
    assert np.all(ex0 == 0) and np.all(tol0 > 0) and np.all(tol0 < 1e-11)
    far = (a + 3) % 6
    _, ex, tol = O.kmeans_assign(x, cent, other=far)
    for h in range(2):
        for n in range(0, 60, 7):
            xn = [Fr(float(v)) for v in x[0, n, h]]
            d = [sum((u - Fr(float(cv))) ** 2 for u, cv in zip(xn, cent[0, h, c])) for c in range(6)]
            want = float(d[far[0, h, n]] - d[a[0, h, n]])
            assert abs(ex[0, h, n] - want) <= 1e-13 * (1 + abs(want))
    assert np.all(ex > tol)
    # an exact tie: token 2 halfway between the two starting centroids; either choice is valid
    xt = np.array([[[2.0, 0.0], [0.0, 2.0], [1.0, 1.0]]], np.float32)[:, :, None, :]
    c0 = O.kmeans_start(xt, 2)
    assert O.kmeans_assign(xt, c0)[0, 0].tolist() == [0, 1, 0]
    _, ext, tolt = O.kmeans_assign(xt, c0, other=np.array([[[0, 1, 1]]], np.int32))
    assert ext[0, 0, 2] == 0 and np.all(ext <= tolt)


def test_kmeans_means_against_exact_means():
    # members' means against exact rational means (one rounding of the exact value
    # apart at most a few ulps of float64 summation), the absolute sums exactly, and an
    # empty cluster keeping its given centroid
    from fractions import Fraction as Fr
    rng = np.random.default_rng(22)
    x = rng.standard_normal((1, 90, 1, 5)).astype(np.float32)
    a = rng.integers(0, 4, size=(1, 1, 90)).astype(np.int32)       # cluster 4 stays empty
    cin = rng.standard_normal((1, 1, 5, 5))
    cent, cnt, sabs = O.kmeans_means(x, a, cin)
    assert cnt[0, 0].tolist() == [int((a == c).sum()) for c in range(5)]
    assert np.array_equal(cent[0, 0, 4], cin[0, 0, 4])
    for c in range(4):
        mem = np.where(a[0, 0] == c)[0]
        for d in range(5):
            ex = sum(Fr(float(x[0, n, 0, d])) for n in mem) / len(mem)
            assert abs(cent[0, 0, c, d] - float(ex)) <= 8 * len(mem) * 2.0 ** -53 * float(sabs[0, 0, c, d]) / len(mem)
            assert sabs[0, 0, c, d] == float(sum(abs(Fr(float(x[0, n, 0, d]))) for n in mem))


def test_kmeans_is_start_then_alternating_steps():
    x = _rand_qkv(1, 80, 2, 8, 23)[0]
    cent = O.kmeans_start(x, 7)
    for it in range(1, 5):
        a = O.kmeans_assign(x, cent)
        cent, cnt, _ = O.kmeans_means(x, a, cent)
        ra, rc, rn = O.kmeans(x, 7, it)
        assert np.array_equal(a, ra) and np.array_equal(cent, rc) and np.array_equal(cnt, rn)


def test_kmeans_equidistant_token_goes_to_the_lower_cluster():
    # token 2 sits exactly halfway between tokens 0 and 1, the starting centroids of
    # clusters 0 and 1 (token floor(c N / C) for N = 3, C = 2): equal squared
    # distances, so it joins cluster 0
    x = np.array([[[2.0, 0.0], [0.0, 2.0], [1.0, 1.0]]], np.float32)[:, :, None, :]
    asg, cent, cnt = O.kmeans(x, 2, 1)
    assert asg[0, 0].tolist() == [0, 1, 0] and cnt[0, 0].tolist() == [2, 1]
    assert cent[0, 0, 0].tolist() == [1.5, 0.5] and cent[0, 0, 1].tolist() == [0.0, 2.0]


def test_cluster_layout_closed_forms():
    rng = np.random.default_rng(4)
    B, H, N, C = 1, 2, 500, 9
    assign = rng.integers(0, C, size=(B, H, N)).astype(np.int32)
    assign[0, 1][assign[0, 1] == 4] = 5                   # an empty cluster
    NB = O.blocks_for(N, C)
    st, off, bc = O.cluster_layout(assign, C, NB)
    for h in range(H):
        cnt = np.bincount(assign[0, h], minlength=C)
        assert np.array_equal(np.diff(off[0, h]), -(-cnt // 64))
        for c in range(C):
            slots = st[0, h, 64 * off[0, h, c]:64 * off[0, h, c + 1]]
            assert np.array_equal(slots[:cnt[c]], np.where(assign[0, h] == c)[0])
            assert np.all(slots[cnt[c]:] == -1)
            nblk = off[0, h, c + 1] - off[0, h, c]
            want = [64] * (nblk - 1) + ([cnt[c] - 64 * (nblk - 1)] if nblk else [])
            assert bc[0, h, off[0, h, c]:off[0, h, c + 1]].tolist() == want
        assert np.all(bc[0, h, off[0, h, C]:] == 0) and np.all(st[0, h, 64 * off[0, h, C]:] == -1)
        real = st[0, h][st[0, h] >= 0]
        assert np.array_equal(np.sort(real), np.arange(N))


def test_cluster_mass_closed_forms():
    rng = np.random.default_rng(5)
    B, H, Cq, Ck, D = 1, 2, 4, 6, 8
    cq = rng.standard_normal((B, H, Cq, D))
    ck = rng.standard_normal((B, H, Ck, D))
    nq = np.array([[[3, 0, 5, 1], [2, 2, 2, 2]]], np.int32)
    nk = np.array([[[10, 0, 20, 5, 5, 60], [1, 1, 1, 1, 1, 1]]], np.int32)
    est = O.cluster_mass(cq, nq, ck, nk, 0.5)
    assert np.all(est[0, 0, 1] == 0)                       # empty query cluster
    assert np.all(est[0, 0, :, 1] == 0)                    # empty key cluster
    live = nq[0] > 0
    assert np.abs(est[0][live].sum(-1) - 1).max() < 1e-12
    # zero query centroids: every key cluster scores the same, so its share is its size
    est0 = O.cluster_mass(np.zeros_like(cq), nq, ck, nk, 0.5)
    assert np.abs(est0[0, 0, 0] - nk[0, 0] / nk[0, 0].sum()).max() < 1e-15
    # a single query/key pair of clusters by hand
    w = nk[0, 1] * np.exp(0.5 * (ck[0, 1] @ cq[0, 1, 2]))
    assert abs(est[0, 1, 2, 3] - w[3] / w.sum()) < 1e-12


def test_cluster_blocks_hand_example():
    # one head, 2 query clusters over blocks [0, 2) and [2, 3), 3 key clusters over
    # blocks [0, 1), [1, 1) (empty) and [1, 4); NB = 5
    qoff = np.array([[[0, 2, 3]]], np.int32)
    koff = np.array([[[0, 1, 1, 4]]], np.int32)
    crow = np.array([0, 2, 3], np.int32)
    ccol = np.array([0, 2, 1], np.int32)
    rp, ci = O.cluster_blocks(crow, ccol, qoff, koff, 5)
    assert _csr_rows(rp, ci) == [[0, 1, 2, 3], [0, 1, 2, 3], [], [], []]


def test_cluster_attention_all_and_single_cluster():
    q, k, v = _rand_qkv(1, 120, 2, 16, 12)
    rng = np.random.default_rng(6)
    qa = rng.integers(0, 4, size=(1, 2, 120)).astype(np.int32)
    ka = rng.integers(0, 5, size=(1, 2, 120)).astype(np.int32)
    # every key cluster kept: dense attention (library routine)
    crow = np.arange(0, 2 * 4 * 5 + 1, 5, dtype=np.int32)
    ccol = np.tile(np.arange(5, dtype=np.int32), 8)
    out = O.cluster_attention(q, k, v, qa, ka, 4, 5, 0.25, crow, ccol)
    assert np.abs(out - _torch_sdpa(q, k, v, 0.25)).max() < 1e-12
    # query cluster 2 of head 1 keeps key cluster 3 only; the others keep nothing
    crow = np.zeros(9, np.int32)
    crow[4 + 2 + 1:] = 1
    out = O.cluster_attention(q, k, v, qa, ka, 4, 5, 0.25, crow, np.array([3], np.int32))
    keys = np.where(ka[0, 1] == 3)[0]
    qs = np.where(qa[0, 1] == 2)[0]
    ref = _torch_sdpa(q[:, qs][:, :, 1:2], k[:, keys][:, :, 1:2], v[:, keys][:, :, 1:2], 0.25)
    assert np.abs(out[0, qs, 1] - ref[0, :, 0]).max() < 1e-12
    others = np.setdiff1d(np.arange(120), qs)
    assert np.all(out[0, others, 1] == 0) and np.all(out[0, :, 0] == 0)
    # the token-subset form returns the same rows
    sel = np.array([qs[0], others[0], 119], np.int32)
    sub = O.cluster_attention(q, k, v, qa, ka, 4, 5, 0.25, crow, np.array([3], np.int32), tokens=sel)
    for h in range(2):
        assert np.array_equal(sub[0, h], out[0, sel, h])


def test_round_bf16_nearest_even():
    """bf16 rounding by hand-worked halfway cases, and against torch's float32 -> bf16
    cast (an independent implementation of the same IEEE rounding) on random and
    extreme values."""
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -(1 + 2.0 ** -8),
                  2.0 ** -130, np.inf, -np.inf, 0.0, 3.3895e38], np.float32)
    want = np.array([1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -1.0], np.float32)
    got = O.round_bf16(x)
    assert np.array_equal(got[:4], want)
    assert np.isposinf(got[5]) and np.isneginf(got[6]) and got[7] == 0.0
    r = np.random.default_rng(3).standard_normal(200000).astype(np.float32)
    r *= np.float32(10.0) ** np.random.default_rng(4).integers(-40, 38, r.size).astype(np.float32)
    r = np.concatenate([r, x])
    ref = torch.from_numpy(r).to(torch.bfloat16).float().numpy()
    assert np.array_equal(O.round_bf16(r), ref, equal_nan=True)


def test_fp8_dequantized_bf16_values():
    """The dequantized tiles the FP8 backward reads: a tile whose largest magnitude is
    448 has scale 1, so its values are e4m3 values themselves, which bf16 holds exactly;
    in general the result is the bf16 rounding of the quantizer's own output."""
    grid, tile = (4, 4, 4), (4, 4, 4)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 64, 1, 8)).astype(np.float32) * 100
    x[0, 5, 0, 3] = 448.0
    xhat, scales = O.fp8_tile_quantize(x, grid, tile)
    assert scales[0, 0, 0] == 1.0
    got = O.fp8_dequantized_bf16(x, grid, tile)
    assert np.array_equal(got, xhat)
    assert np.array_equal(got, np.array([O.e4m3_decode(O.e4m3_encode(v)) for v in x.ravel()],
                                        np.float32).reshape(x.shape))
    y = x * np.float32(0.37)
    yhat, _ = O.fp8_tile_quantize(y, grid, tile)
    assert np.array_equal(O.fp8_dequantized_bf16(y, grid, tile), O.round_bf16(yhat))
