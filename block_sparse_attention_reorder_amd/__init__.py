"""MI355X-native block-sparse attention over 3D-tiled token sequences.

The compute path is libfpsa.so (hand-written gfx950 HIP kernels behind the C ABI in
include/fpsa.h); ``fpsa`` is its ctypes binding and ``pipeline`` sequences the
calls over torch-allocated device buffers. ``synth`` and ``workloads`` describe the
synthetic inputs.
"""

__all__ = ["fpsa", "pipeline", "synth", "workloads", "build"]
