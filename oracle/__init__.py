"""FP64 CPU oracle (test infrastructure only; never imported by the library)."""
from .flce_oracle import *  # noqa: F401,F403
