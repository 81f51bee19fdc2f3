"""CPU oracle of the routed-MoE layer forward. Test infrastructure only (see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
