"""CPU oracle (test infrastructure only; see ``oracle.reference``).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  It shares no code with the HIP library.
"""
from .reference import *  # noqa: F401,F403
from . import reference  # noqa: F401
