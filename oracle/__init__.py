"""CPU oracle of the frame-wise gated delta rule (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  It shares no code with the GPU library.
"""
from . import gdn_oracle, bruteforce  # noqa: F401
