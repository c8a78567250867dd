"""CPU oracle (fp64) for the MoE layer hot path: test infrastructure only.

Only the tests, the smoke check and the CPU-baseline leg of the bench may import
this package; the product path never does.
"""
from . import moe_oracle, mx_oracle  # noqa: F401
