"""Stable Latent MoE layer forward pass on MI355X (gfx950).

The compute path is liblmoe.so (hand-written HIP kernels behind a C ABI,
declared in include/lmoe.h); `lmoe` is its thin ctypes binding.
"""

from . import lmoe  # noqa: F401
from .lmoe import (LmoeError, forward, route, permute, expert_gemm, combine_norm, up,  # noqa: F401
                   make_shape, shape_of, make_weights, workspace_bytes, validate, load_library)
