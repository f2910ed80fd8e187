"""fp64 CPU oracle (test infrastructure; see rkl_oracle)."""
from .rkl_oracle import *  # noqa: F401,F403
from . import rkl_oracle  # noqa: F401
