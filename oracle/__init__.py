"""CPU oracle (fp64 NumPy) for the Hybrid Block.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library's product path.
"""
from .hs2_oracle import *  # noqa: F401,F403
