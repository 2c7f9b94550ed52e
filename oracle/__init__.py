"""Float64 CPU oracle for the dense-layer training path (test infrastructure).

Only the tests, the package smoke check and the bench's CPU-baseline leg may
import this package; the HIP library never does.
"""
from .dense_oracle import *  # noqa: F401,F403
