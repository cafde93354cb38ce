"""fp64 CPU oracle for the H2O chunk step -- test infrastructure only.

Imported by the test suite, the package smoke check and the benchmark's CPU
baseline; never by the GPU library.
"""
from .h2o_oracle import *  # noqa: F401,F403
from .h2o_oracle import __all__  # noqa: F401
