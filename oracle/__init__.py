"""fp64 CPU oracle for one STILL hybrid attention layer (test infrastructure only)."""
from .still_oracle import *  # noqa: F401,F403
