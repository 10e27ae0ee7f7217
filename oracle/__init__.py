"""fp64 CPU oracle for MLA (test infrastructure; see mla_oracle.py header)."""
from .mla_oracle import *  # noqa: F401,F403
from . import mla_oracle  # noqa: F401
