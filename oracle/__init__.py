"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .moe_oracle import *  # noqa: F401,F403
