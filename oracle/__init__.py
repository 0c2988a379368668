"""fp64 CPU oracle for the hybrid attention path.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.
Every function has its parity pinned by tests/test_oracle_pins.py.
"""
from .lizard_oracle import *  # noqa: F401,F403
from .lizard_oracle import __all__  # noqa: F401
