"""CPU oracle (test infrastructure only; see sekv_oracle's header)."""
from . import sekv_oracle  # noqa: F401
