"""fp64 CPU oracle of the TQP routed-expert layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the package smoke check and
by the CPU-baseline leg of bench.py, never by the product path.  It shares no
code with the HIP library or its binding.
"""
from .moe_oracle import *  # noqa: F401,F403
