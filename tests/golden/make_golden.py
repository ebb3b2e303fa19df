"""Write the tiny-workload oracle fixture (tests/golden/tiny_oracle.json).

Calls only the CPU oracle and the seeded input generator; nothing here comes from
the HIP path. Run from the repository root: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from block_sparse_attention_reorder_amd import synth  # noqa: E402
from block_sparse_attention_reorder_amd.workloads import WORKLOADS  # noqa: E402


def main():
    w = WORKLOADS["tiny"]
    q, k, v = synth.make_qkv(w.grid, w.B, w.H, w.D, w.amp, w.sigma, w.seed, bf16=False)
    scale = 1.0 / np.sqrt(w.D)
    M = O.block_mass(q, k, w.grid, w.tile, scale)
    rp, ci = O.select_blocks(M.astype(np.float32))
    out, tok = O.masked_attention(q, k, v, w.grid, w.tile, scale, rp, ci)
    dense = O.dense_attention(q, k, v, scale)
    fix = {
        "workload": "tiny: grid 4x8x8, 4x4x4 tiles, H=1, D=64, amp 0.5, sigma 1, seed 0, float32 inputs",
        "inputs_first": {"q": q[0, 0, 0, :4].tolist(), "k": k[0, 0, 0, :4].tolist(), "v": v[0, 0, 0, :4].tolist()},
        "mass": M[0, 0].tolist(),
        "row_ptr": rp.tolist(),
        "col_idx": ci.tolist(),
        "dense_out_token0": dense[0, 0, 0, :8].tolist(),
        "dense_out_token255": dense[0, 255, 0, :8].tolist(),
        "dense_out_abs_sum": float(np.abs(dense).sum()),
        "masked_out_block3_row5": out[0, 0, 3, 5, :8].tolist(),
        "masked_token_block3_row5": int(tok[0, 0, 3, 5]),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(fix, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
