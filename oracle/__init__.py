"""CPU oracle (test infrastructure only; see tsp_oracle's header)."""
from .tsp_oracle import *  # noqa: F401,F403
