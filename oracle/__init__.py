"""CPU float64 oracle (test infrastructure only; see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
