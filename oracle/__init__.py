"""CPU oracle (test infrastructure only; see dreamer_oracle's header)."""
from .dreamer_oracle import *  # noqa: F401,F403
