"""Test infrastructure: the fp64 CPU oracle of the DiT denoise step.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never calls it.
"""
from .dit_oracle import *  # noqa: F401,F403
from .numerics import *    # noqa: F401,F403
