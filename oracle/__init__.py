"""CPU oracle of the MoE-layer forward pass -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything from this package.  The GPU library and its
Python binding never import it; the product path fails when its HIP library
is missing instead of falling back to this code.

Every function here is pinned by a CPU test to something other than itself
(brute force, closed forms, invariants or special cases); see
``tests/test_oracle.py``.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
from . import request_schedule, switch_policy  # noqa: F401
