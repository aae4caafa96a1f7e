"""Float64 CPU oracle for causal Local Linear Attention (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the HIP library and its binding never do.
"""
from .lla_oracle import *  # noqa: F401,F403
from .lla_oracle import sample_rows  # noqa: F401
from . import lla_oracle_bwd  # noqa: F401  (the gradient of the forward above)
