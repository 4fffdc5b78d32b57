"""fp64 CPU oracle (test infrastructure only; see vdn_oracle's module docstring)."""
from . import vdn_oracle  # noqa: F401
