"""fp64 CPU oracle of the log-mel front end -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package.  The HIP library never does.
"""
from .logmel import *  # noqa: F401,F403
from .logmel import __all__  # noqa: F401
