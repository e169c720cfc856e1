"""Seeded synthetic inputs for the Stable Latent MoE layer.

This package is shared by the tests, the benchmark and the smoke check.  It
holds layer configurations and deterministic random tensors, and nothing of
the layer's own arithmetic: no routing, no GEMM, no activation, no norm.  Both
the HIP path and the CPU oracle receive the very bytes produced here.
"""

from .configs import CONFIGS, LayerConfig, get_config  # noqa: F401
from .inputs import make_inputs, raw_numpy, derive_seed  # noqa: F401
