"""fp64 CPU oracle for causal linear attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  It shares no code with the HIP library.
"""
from .linattn_oracle import *  # noqa: F401,F403
from . import linattn_oracle as core  # noqa: F401
