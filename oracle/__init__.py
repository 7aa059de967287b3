"""CPU oracle for the sparse MoE layer forward.

Test infrastructure only: the test-suite, the smoke check and the benchmark's
CPU-baseline leg are its only users.  The product path never imports it.
"""
from .moe_oracle import *  # noqa: F401,F403
