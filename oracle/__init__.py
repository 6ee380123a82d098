"""CPU FP64 oracle (test infrastructure only; see tq_oracle's header)."""
from .tq_oracle import *  # noqa: F401,F403
from . import tq_oracle  # noqa: F401
