"""CPU fp64 oracle for transform-coded KV-cache compression with compressed-domain decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package: only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may use
it.  It shares no code with the HIP library (``compressed_decode_attention_head_amd``).

Parity pins: every function is pinned by ``tests/test_oracle_pins.py`` against closed
forms, literature values, invariants and brute force.  Functions marked
"parity unpinned" in their docstring have no such pin beyond agreement with the GPU.
"""
from .aatc_oracle import *  # noqa: F401,F403
