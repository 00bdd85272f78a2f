"""CPU oracle for the 4-bit MoE layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library.
"""
from .qmoe_oracle import *  # noqa: F401,F403
from .qmoe_oracle import GROUP  # noqa: F401
