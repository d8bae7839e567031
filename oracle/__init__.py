"""fp64 CPU oracle (test infrastructure; see dspark_oracle)."""
from .dspark_oracle import *  # noqa: F401,F403
from . import dspark_oracle  # noqa: F401
