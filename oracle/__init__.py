"""CPU fp64 oracle for differential attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  The product path never does.
"""

from .diffattn_oracle import *  # noqa: F401,F403
