"""CPU oracle for MLA decode (test infrastructure only; never called by the HIP library)."""
from .mla_oracle import *  # noqa: F401,F403
