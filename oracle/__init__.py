"""CPU oracle of the Inkling MoE feed-forward (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the HIP library.
"""
from .inkling_moe_oracle import *  # noqa: F401,F403
