"""fp64 CPU oracle of the Gated DeltaNet prefill path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.  Parity status of
each function is listed in ``gdn_oracle.c``; every function here is pinned by
the ``-m "not gpu"`` tests in ``tests/test_oracle_*.py``.
"""
from . import gdn_oracle  # noqa: F401
