"""CPU oracle for the paged KV-cache decode path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and
shares no code with it.
"""

from .paged_attention import *  # noqa: F401,F403
from .paged_attention import __all__  # noqa: F401
