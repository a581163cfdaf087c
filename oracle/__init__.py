"""CPU oracle for the LC-VQ hot path (test infrastructure only; see lcvq_oracle)."""
from .lcvq_oracle import *  # noqa: F401,F403
