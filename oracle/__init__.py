"""CPU oracle for the TTQ linear projection -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP product path never does, and
shares no code with it.
"""
from .ttq_oracle import *  # noqa: F401,F403
from .ttq_oracle import overhead_ratio  # noqa: F401
