"""Float64 CPU oracle for the dense-layer training path (test infrastructure).

Only the tests, the package smoke check and the bench's CPU-baseline leg may
import this package; the HIP library never does.
"""
from .dense_oracle import *  # noqa: F401,F403
from .rounding_bands import (U32, act_out_dev, dot_band, dx_band, gamma,  # noqa: F401
                             mlp_forward_bands, relu_kink_band, sum_band, xent_grad_band)
