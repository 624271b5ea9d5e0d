"""Test infrastructure: the fp64 CPU oracle.  Only the tests, the smoke check
and the benchmark's CPU-baseline leg import this package; the library never
does."""
from .diffattn_oracle import *  # noqa: F401,F403
