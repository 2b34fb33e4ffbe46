"""CPU oracle for the MoE layer forward pass.

Test infrastructure only: the test-suite, the package ``smoke()`` check and the
benchmark's CPU-baseline leg are its only users.  The product library never
imports it.
"""
from .moe_oracle import *  # noqa: F401,F403
