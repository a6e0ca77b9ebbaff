"""CPU oracle of the SeKV build step and decode step (test infrastructure).

Only the test suite, the graft entry's smoke check and the bench's CPU-baseline
leg may import this package; the HIP library shares no code with it.
"""
from . import sekv_oracle  # noqa: F401
from .sekv_oracle import *  # noqa: F401,F403
