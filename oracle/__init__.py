"""CPU oracle for the MoE FFN layer forward (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the HIP library never does.
"""
from .moe_oracle import *  # noqa: F401,F403
