"""fp64 CPU oracle of RACE attention -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never does.
"""
from .race_oracle import *  # noqa: F401,F403
from .race_oracle import __all__  # noqa: F401
