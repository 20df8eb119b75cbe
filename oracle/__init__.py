"""CPU float64 oracle for the LoopVQ hot path.

Test infrastructure: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg.  It shares no code with the HIP library.
"""
from .lvq_oracle import *  # noqa: F401,F403
