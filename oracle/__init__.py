"""f64 CPU oracle for the KDA chunked forward (test infrastructure only).

Only tests/, the package smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
from .kda_ref import *  # noqa: F401,F403
