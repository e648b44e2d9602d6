"""CPU oracle (test infrastructure only): plain float64 definition of the routed MoE FFN layer."""
from .moe_oracle import *  # noqa: F401,F403
