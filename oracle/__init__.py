"""fp64 CPU oracle of the sparse MoE layer forward.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
bench's CPU-baseline leg, never by the product path.
"""
from . import moe_oracle, variants  # noqa: F401
