"""CPU fp64 oracle of the vocab-parallel LM head + cross entropy.

TEST INFRASTRUCTURE: imported only by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The product library never imports,
links or calls anything here.
"""
from . import vp_oracle, brute  # noqa: F401
from .vp_oracle import *  # noqa: F401,F403
