"""Plain CPU oracle for the CSA2 decode path.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product package.  It shares no
code with the HIP path.
"""
from .oracle import *  # noqa: F401,F403
