"""CPU oracle for the routed-expert MoE layer -- test infrastructure only.

Imported by the test suite, the package smoke check and the benchmark's
``cpu_baseline`` leg; the product path never imports it.
"""
from .moe_oracle import *  # noqa: F401,F403
