"""CPU oracle for WBMM (test infrastructure only; see wbmm_oracle's header)."""
from .wbmm_oracle import *  # noqa: F401,F403
