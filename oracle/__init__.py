"""CPU oracle for block-wise token dropping (test infrastructure only; see uniprefill_oracle)."""
from .uniprefill_oracle import *  # noqa: F401,F403
