"""CPU oracle for the R-KV compression step — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It shares no code with the HIP library.
"""
from . import rkv_oracle, bruteforce  # noqa: F401
