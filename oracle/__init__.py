"""fp64 CPU oracle for causal Local Linear Attention.  TEST INFRASTRUCTURE ONLY:
imported by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg, never by
the product path."""
from .lla_oracle import lla_row, lla_row_parts, lla_rows, lla_forward, default_workers  # noqa: F401
