"""CPU fp64 oracle (test infrastructure only; see fdl_oracle.py)."""
from .fdl_oracle import *  # noqa: F401,F403
