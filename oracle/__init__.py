"""CPU oracle of the Grok-1 MoE FFN layer (test infrastructure; see grok_moe_oracle.py)."""
from .grok_moe_oracle import *  # noqa: F401,F403
