"""CPU oracle for the paged decode path -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  It shares no code with the HIP library.
"""
from .pkv_oracle import *  # noqa: F401,F403
from . import pkv_oracle  # noqa: F401
