"""CPU oracle for block-sparse attention (test infrastructure only; see oracle.oracle)."""
from .oracle import *  # noqa: F401,F403
from .oracle import TIE_TOL  # noqa: F401
