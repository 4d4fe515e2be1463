"""CPU oracle for the NVFP4 KV-cache hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()``
and by ``bench.py``'s CPU-baseline leg, never by the product package.
"""
from .oracle import *  # noqa: F401,F403
