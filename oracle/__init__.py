"""CPU oracle for the VSA hot path -- test infrastructure only.

Importable by the test suite, the smoke check and the benchmark's CPU-baseline
leg; never by the product path.
"""
from .vsa_oracle import *  # noqa: F401,F403
