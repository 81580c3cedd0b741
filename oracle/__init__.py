"""fp64 CPU oracle (test infrastructure only; see nanokv_oracle)."""
from .nanokv_oracle import *  # noqa: F401,F403
