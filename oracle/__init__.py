"""Float64 CPU oracle for the KVSculpt distillation optimizer.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use this package.  It shares no code with the HIP library.
Every function is pinned by checks in tests/test_oracle_*.py; see the
docstring of oracle.kvsculpt for the list.
"""
from . import kvsculpt  # noqa: F401
