"""fp64 CPU oracle for the sparse-query denoising step (test infrastructure only)."""
from .dlm_oracle import *  # noqa: F401,F403
