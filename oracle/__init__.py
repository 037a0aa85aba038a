"""Float64 CPU oracle for the DoRA hot path.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's CPU-baseline leg may import
this package.  The HIP library never calls it and shares no code with it.
"""
from .dora import *  # noqa: F401,F403
from .dora import __all__  # noqa: F401
