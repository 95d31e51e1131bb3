"""CPU oracle for the Q-GaLore optimizer step (test infrastructure only; never imported by
the product path)."""
from .qgalore_oracle import *  # noqa: F401,F403
