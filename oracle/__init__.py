"""CPU oracle for the streaming-MoE decode path: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never imports, calls or links anything here; the two share no code.
"""
from .reference import *  # noqa: F401,F403
