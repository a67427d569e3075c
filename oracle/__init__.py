"""CPU fp64 oracle for split-KV decode attention (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the HIP library.
"""
from .attention import *  # noqa: F401,F403
from .attention import __all__  # noqa: F401
