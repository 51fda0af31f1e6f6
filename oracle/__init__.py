"""CPU oracle of the gated delta-rule layer step (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library never calls it.
"""
from .oracle import *  # noqa: F401,F403
