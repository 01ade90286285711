"""CPU oracle (test infrastructure only; see fp4lin_oracle's header)."""
from .fp4lin_oracle import *  # noqa: F401,F403
