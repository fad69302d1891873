"""fp64 CPU oracle for paged KV attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline
may import this package.  The product path (the HIP library and its binding)
never calls into it and shares no code with it.
"""
from .paged_oracle import *  # noqa: F401,F403
