"""The CPU oracle and the C ABI's host layer under AddressSanitizer and
UndefinedBehaviorSanitizer.

Each check builds a sanitized copy (the oracle with gcc, the library's host code with
hipcc, device code unchanged) and runs an existing CPU test module against it in a
child process with the matching sanitizer runtime preloaded: the oracle pins
(tests/test_oracle_pins.py, which include out-of-range CSR entries, empty rows and
ragged grids) and the host validation of every ABI call (tests/test_abi_host.py). Any
sanitizer report aborts the child, so the check is its exit status plus the absence
of a report in its output."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_child(env_extra, test_file):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", test_file)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert not any(m in out for m in REPORTS), out[-4000:]
    assert " passed" in out


def test_oracle_pins_under_asan_and_ubsan():
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    env = {"FPSA_ORACLE_SANITIZE": "1"}
    subprocess.run([sys.executable, "-c", "import oracle; oracle.build(force=True)"], cwd=ROOT,
                   env=dict(os.environ, **env), check=True)
    _run_child(dict(env, LD_PRELOAD=f"{asan}:{ubsan}"), "test_oracle_pins.py")


def test_abi_host_layer_under_asan_and_ubsan():
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("the ROCm compiler's sanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from block_sparse_attention_reorder_amd import build
    lib = build.build(verbose=False, sanitize=True)
    _run_child({"LD_PRELOAD": rts[-1], "FPSA_LIB": lib}, "test_abi_host.py")
