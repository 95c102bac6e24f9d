"""CPU float64 oracle for CommVQ (test infrastructure only; see commvq_oracle)."""
from .commvq_oracle import *  # noqa: F401,F403
