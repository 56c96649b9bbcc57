"""fp64 CPU oracle for certified Top-k attention truncation (test infrastructure only).

Only tests/, the smoke entry point and the benchmark's CPU-baseline leg may
import this package; the library never does.
"""
from .ctopk_oracle import *  # noqa: F401,F403
from .ctopk_oracle import NEAR_BOUNDARY_REL  # noqa: F401
