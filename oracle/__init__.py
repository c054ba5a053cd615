"""CPU fp64 oracle of the SquareQ v3 W4 linear layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the device library.
"""
from .sq_oracle import *  # noqa: F401,F403
from . import sq_oracle  # noqa: F401
