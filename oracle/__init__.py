"""CPU oracle (test infrastructure only; see nanospec_oracle's header)."""
from .nanospec_oracle import *  # noqa: F401,F403
from .nanospec_oracle import Sequence_  # noqa: F401
