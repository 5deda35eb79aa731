"""CPU oracle for HAD inference attention (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package; the GPU library never does.
"""
from .had_oracle import *  # noqa: F401,F403
