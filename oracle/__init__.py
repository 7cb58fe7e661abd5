"""The fp64 CPU oracle.  TEST INFRASTRUCTURE ONLY: imported by the tests, the
smoke check and the benchmark's CPU-baseline leg, never by the product path."""
from .cce_oracle import *  # noqa: F401,F403
