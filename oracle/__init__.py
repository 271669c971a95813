"""CPU oracle for chunkwise-parallel causal linear attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  See ``oracle/linattn.py``.
"""
from .linattn import *  # noqa: F401,F403
from . import linattn  # noqa: F401
