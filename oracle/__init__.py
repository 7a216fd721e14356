"""CPU float64 oracle (test infrastructure only; see tsp_oracle.py)."""
from .tsp_oracle import *  # noqa: F401,F403
