"""CPU oracle for SeedLM's decompress-and-multiply path (test infrastructure only).

Only tests, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may
import this package; the product path never does.
"""
from .seedlm_oracle import *  # noqa: F401,F403
from . import seedlm_oracle  # noqa: F401
