"""Plain CPU oracle of the bit-plane top-k decode path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the
HIP library and never imports it.
"""
from .bpk_oracle import *  # noqa: F401,F403
