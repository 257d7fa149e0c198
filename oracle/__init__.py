"""CPU oracle for the FP8 W8A8 NemotronH Mamba2 mixer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (``include/``,
``fp8_w8a8_linear_amd/``) never imports it, and it imports nothing from the
product path.
"""
from .nhm_oracle import *  # noqa: F401,F403
