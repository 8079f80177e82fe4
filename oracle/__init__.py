"""CPU fp64 oracle of the sparse MoE FFN layer -- test infrastructure only.

Only the tests, the smoke check and the bench's cpu_baseline leg use this package.
"""
from .moe_oracle import *  # noqa: F401,F403
