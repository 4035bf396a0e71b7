"""CPU fp64 oracle for exact attention (test infrastructure only).

Imported only by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``.  The GPU library never imports, links or runs it.
"""
from .attention import *  # noqa: F401,F403
from .attention import __all__  # noqa: F401
