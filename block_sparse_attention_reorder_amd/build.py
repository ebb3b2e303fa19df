"""Build libfpsa.so (gfx950) in-tree with hipcc.

Usage: python -m block_sparse_attention_reorder_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfpsa.so")
SOURCES = ["api.hip", "reorder.hip", "mass.hip", "select.hip", "attn.hip", "bwd.hip", "cluster.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-command-line-argument",
]


# The attention and mass kernels never see NaN scores (padding is -inf and every
# -inf case is guarded), so they are built without IEEE NaN-quieting; otherwise each
# max over MFMA results starts with a canonicalising v_max_f32 x, x, x.
# The k-means kernels reproduce a fixed float64 operation order (no fused
# multiply-add), so their file is built with contraction off.
NO_NAN_SOURCES = {"attn.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"],
                  "mass.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"],
                  "cluster.hip": ["-ffp-contract=off"]}


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for the C ABI's host layer
# (argument validation, workspace carving, launch set-up); device code is unchanged.
# Each sanitizer flag applies to the host compilation only.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, build_dir: str, extra=()) -> str:
    obj = os.path.join(build_dir, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *NO_NAN_SOURCES.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    """Build libfpsa.so; with sanitize=True build a host-sanitized copy instead
    (_build/san/libfpsa.so, loaded with the compiler's ASan runtime preloaded)."""
    build_dir = os.path.join(HERE, "_build", "san" if sanitize else "")
    os.makedirs(build_dir, exist_ok=True)
    extra = SANITIZE_FLAGS if sanitize else []
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), SOURCES))
    out = os.path.join(build_dir, "libfpsa.so") if sanitize else LIB
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build()
    sys.exit(0)
