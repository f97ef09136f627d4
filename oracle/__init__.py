"""CPU oracle (float64 NumPy) for the sparse-MoE layer forward.

TEST INFRASTRUCTURE: imported only by tests/, the smoke check and the
benchmark's CPU-baseline leg; the library never imports or calls it.
"""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
