"""CPU oracle (test infrastructure only; see tq_oracle's module docstring)."""
from . import tq_oracle  # noqa: F401
