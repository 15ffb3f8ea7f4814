"""fp64 CPU oracle (test infrastructure only; see relattn_oracle.py)."""
from .relattn_oracle import *  # noqa: F401,F403
