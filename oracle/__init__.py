"""CPU oracle of the TurboQuant path (float64, NumPy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``, never by the library.  Parity status of each function
is listed in ``turboquant``'s header; every function here is pinned by ``-m "not gpu"``
tests against closed forms, textbook values, invariants, brute force or Monte Carlo.
"""
from .turboquant import *  # noqa: F401,F403
