"""CPU oracle for the Mixture-of-Contexts attention layer.

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
may import it. The product path (sparse_chunk_routed_amd) never imports it and shares no code
with it.

Parity pins: every function is pinned by a -m "not gpu" test in tests/test_oracle_*.py against
special cases, closed forms, invariants, library routines and published values. No function
here is "parity unpinned".
"""
from . import moc_oracle, rng  # noqa: F401
