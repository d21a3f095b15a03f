"""CPU oracle for paged decode attention — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package. It shares no code with the HIP library.
"""
from .paged_attention import *  # noqa: F401,F403
from .paged_attention import __all__  # noqa: F401
