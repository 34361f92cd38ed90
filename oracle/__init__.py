"""CPU oracle for the MoE layer forward. Test infrastructure only: imported by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the product path."""
from .moe_oracle import *  # noqa: F401,F403
