"""CPU oracle (test infrastructure): the plain definition the HIP path is checked against.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
"""
from .nf4_oracle import *  # noqa: F401,F403
