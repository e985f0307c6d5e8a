"""fp64 CPU oracle for paged single-token decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or calls
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; the two meet only at the seeded inputs built by ``synth``.
"""
from .attention import *  # noqa: F401,F403
from .kv_write import *  # noqa: F401,F403
