"""fp64 CPU oracle (test infrastructure; see oracle.oracle)."""
from .oracle import *  # noqa: F401,F403
from . import oracle  # noqa: F401
