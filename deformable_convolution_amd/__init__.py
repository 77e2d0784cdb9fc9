"""MI355X-native 1D deformable convolution (DeformConv1d): forward, backward, and
the packed layer whose offsets (and mask) are generated from its input, and
2D modulated deformable convolution (DCNv2).

The compute lives in ``libdc1d.so`` (HIP kernels for gfx950 behind a C ABI
declared in ``include/dc1d.h``); ``deformable_convolution_amd.dc1d`` is the
thin ctypes binding over it.  ``inputs`` holds the seeded synthetic-input
generator.  The library is loaded on first use, so importing the package
never requires a GPU.
"""
from .dc1d import (  # noqa: F401
    Dc1dError,
    backward,
    backward_workspace_bytes,
    debug_positions,
    forward,
    forward_noalloc,
    forward2d,
    library_path,
    load_library,
    output_length,
    packed_forward,
    packed_workspace_bytes,
    plan,
    plan2d,
    resolve_padding,
    status_string,
    workspace_bytes,
    workspace_bytes2d,
)
