"""fp64 CPU oracle for the GQE attention forward pass (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The HIP library and its binding never do.
"""
from .gqe_oracle import *  # noqa: F401,F403
