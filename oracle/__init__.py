"""CPU fp64 oracle for the DPO head path (test infrastructure only; see dpo_oracle)."""
from .dpo_oracle import *  # noqa: F401,F403
from . import dpo_oracle  # noqa: F401
