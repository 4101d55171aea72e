"""fp64 CPU oracle for the BPT layer forward (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the product path never does.
"""
from .bpt_oracle import *  # noqa: F401,F403
