"""fp64 CPU oracle for the SpargeAttention2 hot path (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP library.
"""
from .sa2_oracle import *  # noqa: F401,F403
from . import sa2_oracle  # noqa: F401
