"""CPU oracle of the NVFP4 W4A4 layer (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package; the HIP library never does.
"""
from .nvfp4_oracle import *  # noqa: F401,F403
