"""CPU oracle for the unified-precision FP8 linear layer (test infrastructure only).

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import this package.  The GPU library shares no code with it.
"""
from . import jet_oracle  # noqa: F401
