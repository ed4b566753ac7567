"""CPU oracle package (test infrastructure only; see tq_oracle.py)."""
from . import tq_oracle  # noqa: F401
