"""CPU oracle (test infrastructure only; see lbq_oracle's header)."""
from . import lbq_oracle  # noqa: F401
