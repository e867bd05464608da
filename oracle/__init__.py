"""Float64 CPU oracle (test infrastructure only; see dcp_oracle's header)."""
from .dcp_oracle import *  # noqa: F401,F403
