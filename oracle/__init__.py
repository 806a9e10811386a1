"""CPU oracle (test infrastructure only): see rma_oracle.py."""
from .rma_oracle import *  # noqa: F401,F403
