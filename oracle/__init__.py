"""Plain float64 CPU oracle for XAttention block-sparse prefill.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library and never imports it.
"""

from .xattn_oracle import *  # noqa: F401,F403
