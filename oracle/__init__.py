"""CPU oracle for the ZHA hot path (fp64, NumPy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library or its binding.
"""
from .zha_oracle import *  # noqa: F401,F403
