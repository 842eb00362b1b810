"""fp64 CPU oracle of the grouped-query attention block.

TEST INFRASTRUCTURE ONLY: imported by the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library.
"""
from .gqa_oracle import *  # noqa: F401,F403
from .gqa_oracle import BlockResult, gqa_block, stacked_decode  # noqa: F401
