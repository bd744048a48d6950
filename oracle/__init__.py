"""CPU oracle for the weight-only quantized linear path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and shares no code with it.
"""
from .qlinear_oracle import *  # noqa: F401,F403
