"""The no-allocation selection entry point (fpsa_select_blocks_noalloc, the library's
static device scratch) against fpsa_select_blocks with a caller workspace, through the
C ABI: bit-identical CSR on two calls in a row, the second with fewer rows and blocks
(the scratch then still holds the first call's values), and both equal to the oracle's
selection. Kept last in collection order (a failure here hides no other test)."""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_reorder_amd import fpsa, synth

pytestmark = pytest.mark.gpu


def _both(m):
    R, nb = m.shape
    md = torch.from_numpy(m).to("cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    rp_a, ci_a = torch.full((R + 1,), -7, **i32), torch.full((R * nb,), -7, **i32)
    ws = torch.empty(fpsa.select_workspace_bytes(R, nb), dtype=torch.uint8, device="cuda")
    fpsa.select_blocks(md, R, nb, 99, 100, rp_a, ci_a, ws)
    rp_b, ci_b = torch.full((R + 1,), -9, **i32), torch.full((R * nb,), -9, **i32)
    fpsa.select_blocks_noalloc(md, R, nb, 99, 100, rp_b, ci_b)
    torch.cuda.synchronize()
    nnz = int(rp_a[-1])
    return rp_a.cpu().numpy(), ci_a[:nnz].cpu().numpy(), rp_b.cpu().numpy(), ci_b[:int(rp_b[-1])].cpu().numpy()


def test_noalloc_selection_equals_workspace_selection_twice():
    first = synth.random_mass_rows(7488, 624, seed=624, tie_frac=0.05, zero_frac=0.02)    # 480p rows
    second = synth.random_mass_rows(300, 100, seed=100, tie_frac=0.1, zero_frac=0.2)     # smaller
    for m in (first, second):
        rp_a, ci_a, rp_b, ci_b = _both(m)
        assert np.array_equal(rp_a, rp_b) and np.array_equal(ci_a, ci_b)
        rp_o, ci_o = O.select_blocks(m, 99, 100)
        assert np.array_equal(rp_b, rp_o) and np.array_equal(ci_b, ci_o)


def test_noalloc_selection_rejects_rows_beyond_its_scratch():
    R = fpsa.SELECT_NOALLOC_MAX_ROWS + 1
    m = torch.zeros((1,), dtype=torch.float32, device="cuda")
    rp = torch.empty(1, dtype=torch.int32, device="cuda")
    ci = torch.empty(R * 2, dtype=torch.int32, device="cuda")
    with pytest.raises(fpsa.FpsaError) as e:
        fpsa.select_blocks_noalloc(m, R, 2, 99, 100, rp, ci)
    assert e.value.status == fpsa.ERR_CAPACITY
