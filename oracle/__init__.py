"""CPU oracle for SANTA decode-step attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  See ``oracle/santa.py``.
"""
from . import santa  # noqa: F401
