"""CPU oracle of the MoE layer share (test infrastructure only; see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import default_h_mode  # noqa: F401
