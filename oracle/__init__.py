"""CPU oracle of one DiT denoising step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
The HIP library never routes through this package, and this package imports
nothing from the HIP side (it takes plain numpy arrays).

See ``oracle/dit.py`` for what it computes and where each step comes from.
"""
from .dit import *  # noqa: F401,F403
