"""CPU oracle of the MoE-layer hot path -- test infrastructure only.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the product path.  See moe_oracle.py for the sources it follows.
"""
from . import moe_oracle  # noqa: F401
