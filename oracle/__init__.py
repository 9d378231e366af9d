"""CPU oracle (test infrastructure only; see moe_oracle's header)."""
from .moe_oracle import *  # noqa: F401,F403
