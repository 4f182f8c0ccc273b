"""CPU oracle (test infrastructure only; see dsa_oracle's header)."""
from .dsa_oracle import *  # noqa: F401,F403
from . import dsa_oracle  # noqa: F401
