"""fp64 CPU oracle of the two-tier sparse-attention hot path.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it. The HIP library never calls it, and it shares
no code with the library.
"""
from .oracle import *  # noqa: F401,F403
