"""fp64 CPU oracles for causal Local Linear Attention and for the Parallax forward with a
given probe.  TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg, never by the product path."""
from .lla_oracle import lla_row, lla_row_parts, lla_rows, lla_forward, lla_decode, default_workers  # noqa: F401
from .parallax_oracle import (parallax_row, parallax_row_parts, parallax_rows,  # noqa: F401
                              parallax_forward, parallax_decode, parallax_backward)
