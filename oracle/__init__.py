"""CPU oracle for the BitLinear hot path of BitNet a4.8 -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library never calls it and shares no code with it.
"""
from .bitlinear_oracle import *  # noqa: F401,F403
