"""Float64 CPU oracle for exact attention.  TEST INFRASTRUCTURE ONLY.

Imported only by ``tests/``, by ``__graft_entry__.smoke()`` and by the
benchmark's CPU-baseline leg.  It shares no code with the HIP library.
"""
from .attention import *  # noqa: F401,F403
from .attention import __all__  # noqa: F401
