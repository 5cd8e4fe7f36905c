"""CPU oracle (test infrastructure only; see fp8dq_oracle.py)."""
from .fp8dq_oracle import *  # noqa: F401,F403
from . import fp8dq_oracle as _m

__all__ = [n for n in dir(_m) if not n.startswith("_")]
