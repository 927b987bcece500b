"""CPU oracle for paged decode attention: test infrastructure only.

Imported only by the tests, the smoke check and the benchmark's CPU-baseline
leg; never by the GPU library.
"""
from . import pa_oracle
from .pa_oracle import *  # noqa: F401,F403
