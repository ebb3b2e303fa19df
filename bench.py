"""Benchmark of the whole block-sparse hot path on one MI355X.

One step = tile Q, K (QK operand layout) and V (VT) -> dense block-mass pass -> 99 % retained-mass
selection -> block-sparse forward over the kept blocks -> untile O, on the
Wan2.1-1.3B-shaped 480p workload (grid 21x30x52, 12 heads, head size 128, bf16,
synthetic seeded inputs already resident in HBM).

Prints one JSON line. `value` is kept-block TFLOP per step (nnz * 4 * 64 * 64 * D,
the MFMA work of the sparse forward) divided by the whole step time; per-kernel
times come from HIP events recorded on the stream the kernels run on.

`--workload wan720p | hunyuan720p | grat8192` instead prints per-call timings of that
workload (medians with p10/p90): the 720p step with the FP8 Q/K forward, the
HunyuanVideo dense call followed by ten calls on its frozen selection, or the
8192x8192 image with the fixed structured mask.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "fp8": 5000.0, "fp64": 78.6}   # dense MFMA, TFLOP/s
HBM_PEAK = 8000.0                                # GB/s
CSRC = os.path.join(ROOT, "block_sparse_attention_reorder_amd", "csrc")
# sources each timed kernel is built from (its counters go stale when they change)
KERNEL_SOURCES = {
    "sparse_fwd": ["attn.hip", "attn_common.h", "fpsa_device.h"],
    "sparse_fwd_fp8": ["attn.hip", "attn_common.h", "fpsa_device.h"],
    "block_mass": ["mass.hip", "attn_common.h", "fpsa_device.h"],
    "tile_qkv": ["reorder.hip", "fpsa_device.h"],
    "untile": ["reorder.hip", "fpsa_device.h"],
    "select": ["select.hip", "fpsa_device.h"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload="wan480p"):
    """HBM bytes per call of `kernel` at `workload` from the committed counter runs
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter on a plain copy of known
    size; a call is one launch except for a mass pass in a bounded workspace), or None
    when there is no such run or the kernel's sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get("workloads", {}).get(workload, {}).get("kernels", {}).get(kernel)
    if not e or e.get("source_sha256") != source_hash(kernel):
        return None
    return int(e["hbm_bytes_per_call"])


def algorithmic_bytes(kernel, B, H, D, npad, nb, R, nnz):
    """Bytes a call must move at least: each operand tile read once, each output
    written once (the CSR read once for the forward)."""
    t = B * H * npad * D
    csr = 4 * (R + 1) + 4 * nnz
    if kernel == "sparse_fwd":                      # Q, K, V read, O written, bf16
        return 4 * t * 2 + csr
    if kernel == "sparse_fwd_fp8":                  # e4m3 Q, K and their tile scales; bf16 V, O
        return 2 * t + 2 * t * 2 + 2 * B * H * nb * 4 + csr
    if kernel == "block_mass":                      # Q, K read, float32 masses written
        return 2 * t * 2 + B * H * nb * nb * 4
    raise KeyError(kernel)


def traffic_fields(kernel, workload, B, H, D, npad, nb, R, nnz):
    meas = measured_traffic(kernel, workload)
    alg = algorithmic_bytes(kernel, B, H, D, npad, nb, R, nnz)
    return {"hbm_bytes_measured": meas, "algorithmic_bytes": alg,
            "traffic_ratio": None if meas is None else round(meas / alg, 2)}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="wan480p")
    p.add_argument("--cpu-sample", type=int, default=624,
                   help="query blocks of head 0 the oracle runs for the CPU baseline (0: skip)")
    p.add_argument("--kernels-only", action="store_true", help="skip the CPU baseline")
    p.add_argument("--gemm-reference", action="store_true",
                   help="only time a library bf16 GEMM (torch.matmul, 8192^3 and 16384^3) and the library's dense "
                        "flash attention at the 480p shape: references for the kernels' rates")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="after timing, run one plain 256 MiB device copy (reference for counter runs)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_attention_reorder_amd import synth
    from block_sparse_attention_reorder_amd.pipeline import BlockSparseAttention
    from block_sparse_attention_reorder_amd.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.gemm_reference:
        gemm_reference(dev, args.steps)
        return
    if w.name != "wan480p":
        measure_workload(args, w, dev)
        return
    q, k, v = synth.make_qkv(w.grid, w.B, w.H, w.D, w.amp, w.sigma, w.seed, bf16=True)
    qd, kd, vd = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v))
    bsa = BlockSparseAttention(w.grid, w.tile, w.B, w.H, w.D, device=dev)

    qt = torch.empty(bsa.tiled_shape(), dtype=torch.bfloat16, device=dev)
    kt = torch.empty_like(qt)
    vt = torch.empty_like(qt)
    ot = torch.empty_like(qt)
    o = torch.empty((w.B, bsa.N, w.H, w.D), dtype=torch.bfloat16, device=dev)
    mass = torch.empty((w.B, w.H, bsa.nb, bsa.nb), dtype=torch.float32, device=dev)
    csr = bsa.new_csr()
    ws = bsa.workspace()
    mws = bsa.mass_workspace()
    stream = torch.cuda.current_stream()

    stages = ["tile_qkv", "block_mass", "select", "sparse_fwd", "untile"]

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        bsa.tile_qk(qd, qt)
        bsa.tile_qk(kd, kt)
        bsa.tile_vt(vd, vt)
        if ev is not None:
            ev[1].record(stream)
        bsa.block_mass(qt, kt, mass=mass, workspace=mws)
        if ev is not None:
            ev[2].record(stream)
        bsa.select(mass, 99, 100, csr=csr, workspace=ws)
        if ev is not None:
            ev[3].record(stream)
        bsa.forward(qt, kt, vt, csr, out=ot)
        if ev is not None:
            ev[4].record(stream)
        bsa.untile(ot, out=o)
        if ev is not None:
            ev[5].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nnz = int(csr.row_ptr[-1].item())

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    per = {s: float(np.mean([events[i][j].elapsed_time(events[i][j + 1]) for i in range(args.steps)]))
           for j, s in enumerate(stages)}
    assert int(csr.row_ptr[-1].item()) == nnz

    D, H, B = w.D, w.H, w.B
    kept_flop = nnz * 4.0 * 64 * 64 * D
    mass_flop = 2.0 * bsa.npad * bsa.npad * D * H * B        # one QK^T sweep
    eff_flop = 4.0 * bsa.N * bsa.N * D * H * B           # dense-equivalent over real tokens
    tile_bytes = 3 * (B * bsa.N * H * D * 2 + B * H * bsa.npad * D * 2)
    untile_bytes = B * H * bsa.npad * D * 2 + B * bsa.N * H * D * 2
    select_bytes = 4 * bsa.R * bsa.nb * 2 + 4 * (bsa.R + 1) + 4 * nnz   # mass read twice
    kernels = {
        "sparse_fwd": {"bound": "mfma", "ms": per["sparse_fwd"], "achieved": kept_flop / per["sparse_fwd"] / 1e9,
                       "peak": PEAK["bf16"], "unit": "TFLOP/s", "work_per_unit": "4*64*64*D FLOP per kept block pair",
                       "units": nnz},
        "block_mass": {"bound": "mfma", "ms": per["block_mass"], "achieved": mass_flop / per["block_mass"] / 1e9,
                       "peak": PEAK["bf16"], "unit": "TFLOP/s", "work_per_unit": "2*64*64*D FLOP per block pair (one QK^T sweep)",
                       "units": bsa.R * bsa.nb},
        "tile_qkv": {"bound": "hbm", "ms": per["tile_qkv"], "achieved": tile_bytes / per["tile_qkv"] / 1e6,
                     "peak": HBM_PEAK, "unit": "GB/s", "work_per_unit": "D*2 bytes read + D*2 written per token-head",
                     "units": 3 * B * H * bsa.npad},
        "select": {"bound": "hbm", "ms": per["select"], "achieved": select_bytes / per["select"] / 1e6,
                   "peak": HBM_PEAK, "unit": "GB/s", "work_per_unit": "2*nb*4 bytes read per row + CSR written",
                   "units": bsa.R},
        "untile": {"bound": "hbm", "ms": per["untile"], "achieved": untile_bytes / per["untile"] / 1e6,
                   "peak": HBM_PEAK, "unit": "GB/s", "work_per_unit": "D*2 bytes read + D*2 written per token-head",
                   "units": B * H * bsa.npad},
    }
    for kk in kernels.values():
        kk["frac"] = kk["achieved"] / kk["peak"]
    for name, kk in kernels.items():
        kk["traffic"] = measured_traffic(name)
        if name in ("sparse_fwd", "block_mass"):
            kk.update(traffic_fields(name, w.name, B, H, D, bsa.npad, bsa.nb, bsa.R, nnz))
        elif kk["traffic"] is not None:                # HBM-bound: counter bytes over the timed call
            kk["achieved_GBps_measured"] = round(kk["traffic"] / kk["ms"] / 1e6, 1)
    dominant = max(kernels, key=lambda n: kernels[n]["ms"])
    dk = kernels[dominant]
    roofline = {"kernel": dominant, "bound": dk["bound"], "achieved": round(dk["achieved"], 2),
                "peak": dk["peak"], "unit": dk["unit"], "frac": round(dk["frac"], 4),
                "traffic": dk["traffic"], "traffic_vs_algorithmic": dk.get("traffic_ratio")}

    spread = {s: _stats([events[i][j].elapsed_time(events[i][j + 1]) for i in range(args.steps)])
              for j, s in enumerate(stages)}
    # the same stages with the infinity cache flushed before every step (K and V of
    # this workload, 245 MB, would otherwise stay in the 256 MB cache between steps)
    flushed = _stage_times([(s, fn) for s, fn in zip(stages, stage_fns(bsa, qd, kd, vd, qt, kt, vt, ot, o,
                                                                       mass, csr, ws, mws))],
                           args.steps, stream, flush=_flusher(dev))
    flushed = {s: _stats(x) for s, x in flushed.items()}

    extras = next_rows(bsa, w, qd, kd, qt, kt, vt, ot, mass, csr, stream, max(3, args.steps // 4))

    if args.calibrate_copy:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if args.cpu_sample > 0 and not args.kernels_only:
        cpu = cpu_baseline(w, q, k, v, bsa, args.cpu_sample)

    out = {
        "metric": "block-sparse attn ms/call + kept-block TFLOP/s (% MFMA peak), Wan-1.3B 480p shape",
        "value": round(kept_flop / ms_step / 1e9, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded sinusoidal positional features + N(0,1) noise, bf16",
        "config": {"workload": f"{w.name}: {w.note}", "grid": list(w.grid), "tile": list(w.tile),
                   "batch": w.B, "heads": w.H, "head_dim": w.D, "threshold": "99/100",
                   "nb": bsa.nb, "kept_pairs": nnz, "density": round(nnz / (bsa.R * bsa.nb), 4)},
        "sparse_fwd_ms_per_call": round(per["sparse_fwd"], 4),
        "sparse_fwd_kept_tflops": round(kernels["sparse_fwd"]["achieved"], 2),
        "sparse_fwd_frac_of_bf16_peak": round(kernels["sparse_fwd"]["frac"], 4),
        "sparse_fwd_effective_tflops": round(eff_flop / per["sparse_fwd"] / 1e9, 2),
        "stage_ms": {s: round(x, 4) for s, x in per.items()},
        "stage_ms_spread": spread,
        "stage_ms_flushed": flushed,
        "kernels": {n: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in d.items()}
                    for n, d in kernels.items()},
        "roofline": roofline,
        "next_rows": extras,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def stage_fns(bsa, qd, kd, vd, qt, kt, vt, ot, o, mass, csr, ws, mws):
    """The five stages of the headline step as separate callables."""
    return [lambda: (bsa.tile_qk(qd, qt), bsa.tile_qk(kd, kt), bsa.tile_vt(vd, vt)),
            lambda: bsa.block_mass(qt, kt, mass=mass, workspace=mws),
            lambda: bsa.select(mass, 99, 100, csr=csr, workspace=ws),
            lambda: bsa.forward(qt, kt, vt, csr, out=ot),
            lambda: bsa.untile(ot, out=o)]


def _stats(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "mean": round(float(a.mean()), 4), "n": int(a.size)}


def _flusher(dev):
    """Rewrites a 512 MiB buffer (twice the infinity cache) so that nothing read
    before it is still cached."""
    import torch
    buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    return lambda: buf.zero_()


def _stage_times(stages, reps, stream, flush=None):
    """Runs the (name, fn) stages in order `reps` times, each between HIP events on
    `stream` (flush, when given, runs before each repetition, outside the events).
    Returns name -> list of ms."""
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(reps)]
    for r in range(reps):
        if flush is not None:
            flush()
        evs[r][0].record(stream)
        for i, (_, fn) in enumerate(stages):
            fn()
            evs[r][i + 1].record(stream)
    torch.cuda.synchronize()
    return {name: [evs[r][i].elapsed_time(evs[r][i + 1]) for r in range(reps)] for i, (name, _) in enumerate(stages)}


def device_inputs(w, step, dev, pe):
    """Q, K, V [B, N, H, D] bf16 of call `step` drawn on the device: amp * pe + sigma *
    N(0, 1) with the positional features of the workload and noise from torch's
    generator seeded by (seed, step). Same recipe and distribution as the host
    generator, used where drawing ~10^9 normals on the host would dominate the run."""
    import torch
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 * w.seed + step)
    sigma = w.sigma_at(step)
    base = (pe * w.amp).view(1, w.N, 1, w.D)
    out = []
    for _ in range(3):
        x = torch.randn((w.B, w.N, w.H, w.D), generator=gen, device=dev, dtype=torch.float32)
        x.mul_(sigma).add_(base)
        out.append(x.to(torch.bfloat16))
        del x
    return out


def gemm_reference(dev, reps):
    """Library bf16 GEMM (hipBLASLt through torch.matmul) and dense flash attention on this machine,
    one JSON line each."""
    import torch
    for n in (8192, 16384):
        a = torch.randn(n, n, device=dev).to(torch.bfloat16)
        b = torch.randn(n, n, device=dev).to(torch.bfloat16).t().contiguous()
        c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b, out=c)
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = 2.0 * n ** 3 / ms / 1e9
        print(json.dumps({"gemm": f"bf16 {n}x{n}x{n}, torch.matmul", "ms": round(ms, 4), "tflops": round(tf, 1),
                          "frac_of_bf16_peak": round(tf / PEAK["bf16"], 4)}), flush=True)
        del a, b, c
    # the library's dense FlashAttention at the 480p attention shape (12 heads, 32,760
    # tokens, head size 128, bf16), flash backend only (no fallback to other paths)
    from torch.nn.attention import SDPBackend, sdpa_kernel
    B, H, N, D = 1, 12, 32760, 128
    q, k, v = (torch.randn(B, H, N, D, device=dev).to(torch.bfloat16) for _ in range(3))
    try:
        with sdpa_kernel(SDPBackend.FLASH_ATTENTION):
            fn = lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v)
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            e1.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = 4.0 * N * N * D * H * B / ms / 1e9
        print(json.dumps({"attention": f"dense bf16 B={B} H={H} N={N} D={D}, torch scaled_dot_product_attention "
                                       f"(flash backend)", "ms": round(ms, 4), "tflops": round(tf, 1),
                          "frac_of_bf16_peak": round(tf / PEAK["bf16"], 4)}), flush=True)
    except RuntimeError as err:
        print(json.dumps({"attention": "flash backend unavailable", "error": str(err)[:200]}), flush=True)


def _kernel_entry(times, flop=None, peak=None, nbytes=None):
    e = _stats(times)
    if flop is not None:
        e["achieved_tflops"] = round(flop / e["median"] / 1e9, 2)
        e["frac_of_peak"] = round(flop / e["median"] / 1e9 / peak, 4)
        e["peak_tflops"] = peak
    if nbytes is not None:
        e["achieved_GBps"] = round(nbytes / e["median"] / 1e6, 1)
        e["frac_of_hbm_peak"] = round(nbytes / e["median"] / 1e6 / HBM_PEAK, 4)
    return e


def measure_workload(args, w, dev):
    """Per-call timings of the larger configurations (one JSON line): Wan2.1-14B 720p
    (bf16 path and the FP8 Q/K forward on the bf16 selection), HunyuanVideo 720p (one
    dense selection step, then ten calls on the frozen CSR) and the 8192x8192 image with
    the fixed structured mask. Medians with p10/p90 over HIP-event timings."""
    import torch
    from block_sparse_attention_reorder_amd import synth
    from block_sparse_attention_reorder_amd.pipeline import BlockSparseAttention

    stream = torch.cuda.current_stream()
    pe = torch.from_numpy(synth.positional_features(w.grid, w.D)).to(dev)
    bsa = BlockSparseAttention(w.grid, w.tile, w.B, w.H, w.D, device=dev)
    D, H, B = w.D, w.H, w.B
    qd, kd, vd = device_inputs(w, 0, dev, pe)
    qt, kt, vt, ot = (torch.empty(bsa.tiled_shape(), dtype=torch.bfloat16, device=dev) for _ in range(4))
    o = torch.empty((B, bsa.N, H, D), dtype=torch.bfloat16, device=dev)
    reps, warm = args.steps, args.warmup
    tile_bytes = 3 * (B * bsa.N * H * D * 2 + B * H * bsa.npad * D * 2)
    untile_bytes = B * H * bsa.npad * D * 2 + B * bsa.N * H * D * 2
    kern = {}
    extra = {}

    def tile_all():
        bsa.tile_qk(qd, qt), bsa.tile_qk(kd, kt), bsa.tile_vt(vd, vt)

    if w.mask == "grat":
        t_build = []
        for _ in range(warm + reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            csr = bsa.structured()
            e1.record(stream)
            torch.cuda.synchronize()
            t_build.append(e0.elapsed_time(e1))
        kern["structured_mask"] = _kernel_entry(t_build[warm:])
        stages = [("tile_qkv", tile_all), ("sparse_fwd", lambda: bsa.forward(qt, kt, vt, csr, out=ot)),
                  ("untile", lambda: bsa.untile(ot, out=o))]
        _stage_times(stages, warm, stream)
        t = _stage_times(stages, reps, stream)
        nnz = int(csr.row_ptr[-1].item())
        kept = nnz * 4.0 * 64 * 64 * D
        kern["tile_qkv"] = _kernel_entry(t["tile_qkv"], nbytes=tile_bytes)
        kern["sparse_fwd"] = _kernel_entry(t["sparse_fwd"], kept, PEAK["bf16"])
        kern["untile"] = _kernel_entry(t["untile"], nbytes=untile_bytes)
        call_ms = sum(kern[s]["median"] for s in ("tile_qkv", "sparse_fwd", "untile"))
        value = kept / call_ms / 1e9
        what = "tile Q, K, V -> sparse forward over the fixed structured mask -> untile O"
    else:
        mass = torch.empty((B, H, bsa.nb, bsa.nb), dtype=torch.float32, device=dev)
        csr = bsa.new_csr()
        ws = bsa.workspace()
        mws = bsa.mass_workspace()
        stages = list(zip(["tile_qkv", "block_mass", "select", "sparse_fwd", "untile"],
                          stage_fns(bsa, qd, kd, vd, qt, kt, vt, ot, o, mass, csr, ws, mws)))
        _stage_times(stages, warm, stream)
        nreps = reps if w.reuse_steps == 0 else max(3, reps // 4)
        t = _stage_times(stages, nreps, stream)
        nnz = int(csr.row_ptr[-1].item())
        kept = nnz * 4.0 * 64 * 64 * D
        mass_flop = 2.0 * bsa.npad * bsa.npad * D * H * B
        kern["tile_qkv"] = _kernel_entry(t["tile_qkv"], nbytes=tile_bytes)
        kern["block_mass"] = _kernel_entry(t["block_mass"], mass_flop, PEAK["bf16"])
        kern["select"] = _kernel_entry(t["select"])
        kern["sparse_fwd"] = _kernel_entry(t["sparse_fwd"], kept, PEAK["bf16"])
        kern["untile"] = _kernel_entry(t["untile"], nbytes=untile_bytes)
        step_ms = sum(kern[s]["median"] for s in ("tile_qkv", "block_mass", "select", "sparse_fwd", "untile"))
        value = kept / step_ms / 1e9
        what = "tile Q, K, V -> mass pass -> 99 % selection -> sparse forward -> untile O"
        if w.fp8:
            q8, k8 = (torch.empty(bsa.tiled_shape(), dtype=torch.uint8, device=dev) for _ in range(2))
            qs, ks = (torch.empty((B, H, bsa.nb), dtype=torch.float32, device=dev) for _ in range(2))
            st8 = [("tile_qk_fp8", lambda: (bsa.tile_fp8(qd, q8, qs), bsa.tile_fp8(kd, k8, ks))),
                   ("sparse_fwd_fp8", lambda: bsa.forward(q8, k8, vt, csr, q_scale=qs, k_scale=ks, out=ot))]
            _stage_times(st8, warm, stream)
            t8 = _stage_times(st8, reps, stream)
            # QK^T at the fp8 rate and P*V at the bf16 rate: 4 FLOP units per pair take
            # 2/fp8 + 2/bf16 time units
            mixed = 4.0 / (2.0 / PEAK["fp8"] + 2.0 / PEAK["bf16"])
            fp8_bytes = 2 * (B * bsa.N * H * D * 2 + B * H * bsa.npad * D) + 2 * B * H * bsa.nb * 4
            kern["tile_qk_fp8"] = _kernel_entry(t8["tile_qk_fp8"], nbytes=fp8_bytes)
            e = _kernel_entry(t8["sparse_fwd_fp8"], kept, mixed)
            e["frac_of_fp8_peak"] = round(kept / e["median"] / 1e9 / PEAK["fp8"], 4)
            e["peak_note"] = "mixed peak: QK^T at 5.0 PFLOP/s fp8, P*V at 2.5 PFLOP/s bf16"
            kern["sparse_fwd_fp8"] = e
        if w.reuse_steps:
            # one dense selection call (above), then calls 1..reuse_steps with their own
            # inputs on the frozen CSR
            one_time = kern["block_mass"]["median"] + kern["select"]["median"]
            calls = [kern["tile_qkv"]["median"] + kern["sparse_fwd"]["median"] + kern["untile"]["median"]]
            fwd = []
            st = [("tile_qkv", tile_all), ("sparse_fwd", lambda: bsa.forward(qt, kt, vt, csr, out=ot)),
                  ("untile", lambda: bsa.untile(ot, out=o))]
            for s in range(1, w.reuse_steps + 1):
                del qd, kd, vd
                qd, kd, vd = device_inputs(w, s, dev, pe)
                _stage_times(st, 1, stream)
                ts = _stage_times(st, 3, stream)
                med = {k_: sorted(v_)[1] for k_, v_ in ts.items()}
                fwd.append(med["sparse_fwd"])
                calls.append(sum(med.values()))
            extra["frozen_calls"] = {
                "sparse_fwd_ms_per_call": [round(x, 4) for x in fwd],
                "sparse_fwd_mean_ms": round(sum(fwd) / len(fwd), 4),
                "sparse_fwd_mean_tflops": round(kept / (sum(fwd) / len(fwd)) / 1e9, 2),
                "one_time_mass_and_select_ms": round(one_time, 4),
                "call_ms_amortised_over_%d_calls" % len(calls): round((one_time + sum(calls)) / len(calls), 4),
            }
            value = kept / ((one_time + sum(calls)) / len(calls)) / 1e9
            what = (f"call 0: tile -> mass pass -> 99 % selection -> sparse forward -> untile; calls "
                    f"1..{w.reuse_steps}: tile -> sparse forward on the frozen CSR -> untile; value over the "
                    f"amortised call")
            step_ms = (one_time + sum(calls)) / len(calls)
    for name in ("block_mass", "sparse_fwd", "sparse_fwd_fp8"):
        if name in kern:
            kern[name].update(traffic_fields(name, w.name, B, H, D, bsa.npad, bsa.nb, bsa.R, nnz))
    for name in ("tile_qkv", "select", "untile"):       # HBM-bound: counter bytes over the timed call
        if name in kern:
            tb = measured_traffic(name, w.name)
            kern[name]["hbm_bytes_measured"] = tb
            kern[name]["measured_GBps"] = None if tb is None else round(tb / kern[name]["median"] / 1e6, 1)
    eff_flop = 4.0 * bsa.N * bsa.N * D * H * B          # dense-equivalent over real tokens
    for name in ("sparse_fwd", "sparse_fwd_fp8"):
        if name in kern:
            kern[name]["effective_tflops"] = round(eff_flop / kern[name]["median"] / 1e9, 2)
    out = {
        "metric": f"kept-block TFLOP/s per call, {w.name}",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": warm,
        "ms_per_step": round(kept / value / 1e9, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: positional features + N(0,1) noise drawn on the device (seeded), bf16",
        "config": {"workload": f"{w.name}: {w.note}", "grid": list(w.grid), "tile": list(w.tile), "batch": B,
                   "heads": H, "head_dim": D, "nb": bsa.nb, "kept_pairs": nnz,
                   "density": round(nnz / (bsa.R * bsa.nb), 4), "call": what},
        "kernels_ms": kern,
    }
    out.update(extra)
    if args.cpu_sample > 0 and not args.kernels_only:
        # the oracle on head 0 of the same (device-drawn) inputs, copied to the host;
        # the sample is sized for 10-30 s of host work at this workload's token count
        sample = min(args.cpu_sample, CPU_SAMPLE_BLOCKS.get(w.name, args.cpu_sample))
        if w.reuse_steps:
            qd, kd, vd = device_inputs(w, 0, dev, pe)
        q0, k0, v0 = (x[:, :, :1, :].float().cpu().numpy() for x in (qd, kd, vd))
        out["cpu_baseline"] = cpu_baseline(w, q0, k0, v0, bsa, sample, structured=w.mask == "grat")
    print(json.dumps(out))


# Query blocks of head 0 the CPU baseline samples per workload (the mass pass costs
# O(N) per query block; the structured mask's rows keep about 131 blocks each).
CPU_SAMPLE_BLOCKS = {"wan720p": 256, "hunyuan720p": 160, "grat8192": 2048, "tiny": 4}


def _timed(fn, stream, reps):
    import torch
    fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(reps):
        fn()
    ev[1].record(stream)
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


def next_rows(bsa, w, qd, kd, qt, kt, vt, ot, mass, csr, stream, reps):
    """Timings of the rows beyond the headline path on the same inputs, after the
    timed region: the retained-mass monitor over the step's masses and CSR, and
    fixed per-head patterns (mask build and the forward over them)."""
    import torch
    kept = torch.empty((w.B, w.H, bsa.nb), dtype=torch.float32, device=qt.device)
    nnz = int(csr.row_ptr[-1].item())
    t_mon = _timed(lambda: bsa.retained_mass(mass, csr, out=kept), stream, reps)
    mon_bytes = bsa.R * bsa.nb * 4 + (bsa.R + 1) * 4 + nnz * 4 + bsa.R * 4
    per = bsa.frame_period()
    cycle = [(2, 0, 0, 0), (1, per, 0, 0), (-1, 0, 8, 0), (1, per, 4, 0)]
    pats = [cycle[h % len(cycle)] for h in range(w.H)]
    pcsr = bsa.pattern(pats)
    ws = bsa.workspace()
    patt = torch.as_tensor(pats, dtype=torch.int32).to(qt.device)
    from block_sparse_attention_reorder_amd import fpsa
    t_build = _timed(lambda: fpsa.pattern_mask(bsa.grid, bsa.tile, bsa.B, bsa.H, patt, pcsr.row_ptr,
                                               pcsr.col_idx, ws), stream, reps)
    pnnz = int(pcsr.row_ptr[-1].item())
    t_pf = _timed(lambda: bsa.forward(qt, kt, vt, pcsr, out=ot), stream, reps)
    pflop = pnnz * 4.0 * 64 * 64 * w.D
    # backward over the step's CSR: delta/lse preprocessing, dK/dV per key block,
    # dQ per query block; the transpose is built once per frozen CSR (timed apart)
    lse = torch.empty((w.B, w.H, bsa.npad), dtype=torch.float32, device=qt.device)
    o32 = torch.empty(bsa.tiled_shape(), dtype=torch.float32, device=qt.device)
    bsa.forward(qt, kt, vt, csr, out=ot, lse=lse, out_f32=o32)
    vq = torch.empty_like(qt)
    gt = torch.empty_like(qt)
    gen = torch.Generator(device=qt.device)
    gen.manual_seed(7)
    vq.copy_(torch.randn(qt.shape, generator=gen, device=qt.device, dtype=torch.float32))
    gt.copy_(torch.randn(qt.shape, generator=gen, device=qt.device, dtype=torch.float32))
    csc = bsa.transpose(csr)
    t_tr = _timed(lambda: bsa.transpose(csr), stream, reps)
    grads = tuple(torch.empty_like(qt) for _ in range(3))
    bws = torch.empty(fpsa.bwd_workspace_bytes(w.B, w.H, w.grid, w.tile), dtype=torch.uint8, device=qt.device)
    t_bwd = _timed(lambda: bsa.backward(qt, kt, vq, o32, gt, lse, csr, csc, grads=grads, workspace=bws),
                   stream, reps)
    bflop = nnz * 10.0 * 64 * 64 * w.D          # five 64x64xD products per kept pair
    # backward of the FP8 Q/K forward over the same CSR: Q and K as e4m3 code values in
    # bf16 with the tile scales, lse and float32 output from the FP8 forward
    q8, qs = bsa.tile_fp8(qd)
    k8, ks = bsa.tile_fp8(kd)
    lse8 = torch.empty_like(lse)
    o32f = torch.empty_like(o32)
    bsa.forward(q8, k8, vt, csr, q_scale=qs, k_scale=ks, out=ot, lse=lse8, out_f32=o32f)
    qc, kc = bsa.dequantize(q8, None), bsa.dequantize(k8, None)
    t_codes = _timed(lambda: (bsa.dequantize(q8, None, out=qc), bsa.dequantize(k8, None, out=kc)), stream, reps)
    t_bwd8 = _timed(lambda: bsa.backward(qc, kc, vq, o32f, gt, lse8, csr, csc, grads=grads, workspace=bws,
                                         q_scale=qs, k_scale=ks), stream, reps)
    sem = semantic_row(bsa, w, qt, stream, reps)
    return {
        "retained_mass": {"ms": round(t_mon, 4), "bound": "hbm",
                          "achieved_GBps": round(mon_bytes / t_mon / 1e6, 1),
                          "frac": round(mon_bytes / t_mon / 1e6 / HBM_PEAK, 4),
                          "work_per_unit": "nb*4 bytes of masses + CSR entries per row",
                          "min": round(float(kept.min()), 5), "mean": round(float(kept.mean()), 5)},
        "pattern_mask": {"ms_build": round(t_build, 4), "patterns": "per head, cycling diagonal band 2; "
                         "multi-diagonal band 1 period nh*nw; stripe 8; multi-diagonal + stripe 4",
                         "kept_pairs": pnnz, "density": round(pnnz / (bsa.R * bsa.nb), 4),
                         "fwd_ms": round(t_pf, 4), "fwd_kept_tflops": round(pflop / t_pf / 1e9, 2),
                         "fwd_frac_of_bf16_peak": round(pflop / t_pf / 1e9 / PEAK["bf16"], 4)},
        "backward": {"ms": round(t_bwd, 4), "kept_pairs": nnz,
                     "work_per_unit": "10*64*64*D FLOP per kept pair (QK^T, dO V^T, P^T dO, dS^T Q, dS K)",
                     "tflops": round(bflop / t_bwd / 1e9, 2),
                     "frac_of_bf16_peak": round(bflop / t_bwd / 1e9 / PEAK["bf16"], 4),
                     "transpose_ms": round(t_tr, 4),
                     "inputs": "Q, K from the step; V (QK layout) and dO random normal bf16",
                     "fp8": {"ms": round(t_bwd8, 4), "code_tiles_ms": round(t_codes, 4),
                             "tflops": round(bflop / t_bwd8 / 1e9, 2),
                             "frac_of_bf16_peak": round(bflop / t_bwd8 / 1e9 / PEAK["bf16"], 4),
                             "what": "backward of the FP8 Q/K forward: e4m3 code values of Q and K in bf16 "
                                     "with the tile scales (straight-through quantizer)"}},
        "semantic_permutation": sem,
    }


def semantic_row(bsa, w, qt, stream, reps):
    """k-means semantic permutation at the same shape: 128 query and 128 key clusters,
    4 Lloyd steps, top-90 % clusters; per-stage times and the forward over the
    cluster blocks."""
    import torch
    from block_sparse_attention_reorder_amd import fpsa, synth
    from block_sparse_attention_reorder_amd.pipeline import SemanticSparseAttention
    q, k, v = synth.make_qkv(w.grid, w.B, w.H, w.D, w.amp, w.sigma, w.seed, bf16=True)
    qd, kd, vd = (torch.from_numpy(x).to(qt.device).to(torch.bfloat16) for x in (q, k, v))
    ssa = SemanticSparseAttention(bsa.N, w.B, w.H, w.D, 128, 128, iters=4, device=qt.device)
    qc, kc = ssa.cluster(qd, 128), ssa.cluster(kd, 128)
    st = {}
    st["kmeans_q_and_k"] = _timed(lambda: (ssa.cluster(qd, 128), ssa.cluster(kd, 128)), stream, reps)
    st["gather_qkv"] = _timed(lambda: (ssa.gather(qd, qc, fpsa.LAYOUT_QK), ssa.gather(kd, kc, fpsa.LAYOUT_QK),
                                       ssa.gather(vd, kc, fpsa.LAYOUT_VT)), stream, reps)
    qt2, kt2, vt2 = ssa.gather(qd, qc, fpsa.LAYOUT_QK), ssa.gather(kd, kc, fpsa.LAYOUT_QK), ssa.gather(vd, kc, fpsa.LAYOUT_VT)
    est = ssa.cluster_mass(qc, kc)
    ccsr = ssa.select_clusters(est)
    st["mass_select_blocks"] = _timed(lambda: ssa.block_csr(ssa.select_clusters(ssa.cluster_mass(qc, kc)), qc, kc),
                                      stream, reps)
    csr = ssa.block_csr(ccsr, qc, kc)
    ot = torch.empty(ssa.tiled_shape(), dtype=torch.bfloat16, device=qt.device)
    st["forward"] = _timed(lambda: ssa.forward(qt2, kt2, vt2, kc, csr, out=ot), stream, reps)
    st["scatter"] = _timed(lambda: ssa.scatter(ot, qc), stream, reps)
    nnz = int(csr.row_ptr[-1].item())
    real_pairs = float((kc.blk_count.double().sum() / 64).item())
    flop = nnz * 4.0 * 64 * 64 * w.D
    return {"clusters": [128, 128], "kmeans_steps": 4, "top_p": "90/100",
            "stage_ms": {kk: round(vv, 4) for kk, vv in st.items()},
            "total_ms": round(sum(st.values()), 4),
            "blocks_per_head": ssa.NB, "kept_pairs": nnz,
            "density_of_padded_pairs": round(nnz / (w.B * w.H * ssa.NB * ssa.NB), 4),
            "padding_overhead": round(w.B * w.H * ssa.NB / max(real_pairs, 1.0), 4),
            "fwd_kept_tflops": round(flop / st["forward"] / 1e9, 2),
            "fwd_frac_of_bf16_peak": round(flop / st["forward"] / 1e9 / PEAK["bf16"], 4),
            # the assignment products (2 N C D FLOP per step, slice and tensor, float64
            # MFMA) over the whole k-means time (layout and member lists included)
            "kmeans_fp64_tflops": round(2 * 4 * 2.0 * bsa.N * 128 * w.D * w.B * w.H / st["kmeans_q_and_k"] / 1e9, 2),
            "kmeans_frac_of_fp64_peak": round(2 * 4 * 2.0 * bsa.N * 128 * w.D * w.B * w.H / st["kmeans_q_and_k"]
                                              / 1e9 / PEAK["fp64"], 4)}


def cpu_baseline(w, q, k, v, bsa, nsample, structured=False):
    """The oracle, as it stands, on a bounded sample: mass pass, selection and masked
    attention for `nsample` query blocks of head 0 (first, last and seeded others); on
    the structured-mask workload the fixed mask's rows replace mass pass and selection.
    Reported in the same unit as `value`: kept-block FLOP of the sampled rows over the
    oracle's time for those rows."""
    import numpy as np

    import oracle as O

    rng = np.random.default_rng(12345)
    nb = bsa.nb
    nsample = min(nsample, nb)
    picks = sorted(set([0, nb - 1] + rng.choice(nb, size=max(0, nsample - 2), replace=False).tolist()))[:nsample]
    q0, k0, v0 = (np.ascontiguousarray(x[:, :, :1, :]) for x in (q, k, v))
    t0 = time.perf_counter()
    if structured:
        nh, nw = -(-w.grid[1] // w.tile[1]), -(-w.grid[2] // w.tile[2])
        rp_all, ci_all = O.structured_mask(nh, nw, 1)
        rp_s = np.concatenate([[0], np.cumsum([rp_all[b + 1] - rp_all[b] for b in picks])]).astype(np.int32)
        ci_s = np.concatenate([ci_all[rp_all[b]:rp_all[b + 1]] for b in picks]).astype(np.int32)
        t1 = t2 = time.perf_counter()
    else:
        m = O.block_mass(q0, k0, w.grid, w.tile, bsa.scale, qblocks=picks)
        t1 = time.perf_counter()
        rows = m.reshape(len(picks), nb).astype(np.float32)
        rp_s, ci_s = O.select_blocks(rows)
        t2 = time.perf_counter()
    # expand the sampled rows into a CSR over all rows of head 0 (others empty)
    rp = np.zeros(nb + 1, np.int32)
    counts = np.zeros(nb, np.int64)
    for i, qb in enumerate(picks):
        counts[qb] = rp_s[i + 1] - rp_s[i]
    rp[1:] = np.cumsum(counts)
    ci = ci_s if len(ci_s) else np.zeros(1, np.int32)        # picks are ascending
    O.masked_attention(q0, k0, v0, w.grid, w.tile, bsa.scale, rp, ci, qblocks=picks)
    t3 = time.perf_counter()
    kept = int(len(ci_s))
    flop = kept * 4.0 * 64 * 64 * w.D
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(flop / (t3 - t0) / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(picks)} query blocks of head 0 of {w.name} (first, last, seeded others): "
                      + (f"fixed structured mask rows, masked attention {t3 - t2:.2f} s" if structured else
                         f"float64 mass pass {t1 - t0:.2f} s, selection {t2 - t1:.3f} s, masked attention "
                         f"{t3 - t2:.2f} s") + f"; {kept} kept pairs",
            "seconds": round(t3 - t0, 3)}


if __name__ == "__main__":
    main()
