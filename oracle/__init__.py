"""fp64 CPU oracle for BDLM masked attention.  TEST INFRASTRUCTURE ONLY: only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it."""
from .bdlm_oracle import *  # noqa: F401,F403
