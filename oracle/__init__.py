"""fp64 CPU oracle of the Stable Latent MoE layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's cpu_baseline leg, never by the product path.
"""

from . import lmoe_oracle  # noqa: F401
from .lmoe_oracle import forward  # noqa: F401
