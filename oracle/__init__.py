"""CPU oracle of the TurboQuant KV-cache codec.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library. See tq_oracle.py.
"""
from .tq_oracle import *  # noqa: F401,F403
from .tq_oracle import requantize_key, value_rows, VALUE_BLOCK  # noqa: F401
