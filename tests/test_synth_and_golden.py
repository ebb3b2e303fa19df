"""Seeded generator determinism and the tiny-workload oracle regression fixture."""
import json
import os

import numpy as np

import oracle as O
from block_sparse_attention_reorder_amd import synth
from block_sparse_attention_reorder_amd.workloads import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_oracle.json")


def test_generator_is_deterministic_and_shaped():
    a = synth.make_qkv((3, 4, 8), 2, 3, 16, 1.0, 1.0, 5, bf16=True)
    b = synth.make_qkv((3, 4, 8), 2, 3, 16, 1.0, 1.0, 5, bf16=True)
    for x, y in zip(a, b):
        assert x.shape == (2, 96, 3, 16) and x.dtype == np.float32
        assert np.array_equal(x, y)
    c = synth.make_qkv((3, 4, 8), 2, 3, 16, 1.0, 1.0, 6, bf16=True)
    assert not np.array_equal(a[0], c[0])


def test_generator_bf16_values_are_representable():
    q, _, _ = synth.make_qkv((2, 4, 4), 1, 2, 8, 1.0, 1.0, 0, bf16=True)
    bits = q.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)


def test_positional_features_values():
    pe = synth.positional_features((4, 8, 8), 64)
    # token 0 sits at the origin: sin 0 = 0, cos 0 = 1 on every pair
    assert np.array_equal(pe[0, 0::2], np.zeros(32, np.float32))
    assert np.array_equal(pe[0, 1::2], np.ones(32, np.float32))
    # token (t=0, h=0, w=1): pair i varies only when i mod 3 == 2 (the w axis)
    n = 1
    assert np.isclose(pe[n, 4], np.sin(10000.0 ** (-4 / 64)), atol=1e-7)
    assert pe[n, 0] == 0.0 and pe[n, 2] == 0.0
    pe2 = synth.positional_features((1, 8, 8), 16)        # 2D: axes alternate h, w
    assert pe2[1, 0] == 0.0 and np.isclose(pe2[1, 2], np.sin(10000.0 ** (-2 / 16)), atol=1e-7)


def test_random_mass_rows_have_ties_and_zeros():
    m = synth.random_mass_rows(50, 64, seed=1)
    assert m.dtype == np.float32 and m.shape == (50, 64) and m.min() >= 0
    assert np.any(m == 0)
    assert any(len(np.unique(r[r > 0])) < np.count_nonzero(r) for r in m)


def test_tiny_workload_matches_fixture():
    fix = json.load(open(GOLDEN))
    w = WORKLOADS["tiny"]
    q, k, v = synth.make_qkv(w.grid, w.B, w.H, w.D, w.amp, w.sigma, w.seed, bf16=False)
    assert np.allclose(q[0, 0, 0, :4], fix["inputs_first"]["q"], rtol=0, atol=0)
    scale = 1.0 / np.sqrt(w.D)
    M = O.block_mass(q, k, w.grid, w.tile, scale)
    assert np.abs(M[0, 0] - np.array(fix["mass"])).max() < 1e-12
    rp, ci = O.select_blocks(M.astype(np.float32))
    assert rp.tolist() == fix["row_ptr"] and ci.tolist() == fix["col_idx"]
    out, tok = O.masked_attention(q, k, v, w.grid, w.tile, scale, rp, ci)
    assert int(tok[0, 0, 3, 5]) == fix["masked_token_block3_row5"]
    assert np.abs(out[0, 0, 3, 5, :8] - np.array(fix["masked_out_block3_row5"])).max() < 1e-12
