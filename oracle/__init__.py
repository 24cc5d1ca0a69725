"""fp64 CPU oracle of the MISA indexer (test infrastructure only; see misa_oracle)."""
from .misa_oracle import *  # noqa: F401,F403
