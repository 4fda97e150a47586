"""CPU oracle for the MegaMoE expert layer — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package; the product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
