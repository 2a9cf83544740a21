"""CPU oracle for KATA (test infrastructure only; see kata_oracle.py)."""
from .kata_oracle import *  # noqa: F401,F403
