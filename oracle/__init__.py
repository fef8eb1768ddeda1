"""CPU oracle for the W8A8 INT8 linear layer -- test infrastructure only.

Imported by the tests, by the smoke check and by the benchmark's CPU
baseline; never by the product path.
"""
from .pdq_oracle import *  # noqa: F401,F403
