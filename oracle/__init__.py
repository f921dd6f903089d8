"""Plain fp64 CPU oracle for the CSA/HCA compressed-attention hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path
(the HIP library and its Python binding) never calls it, and this package
shares no code with that path: no kernels, headers, helpers, tables or
constant generators.

Every function restates, in numpy float64, what the pages define; see the
docstrings of ``oracle.dlc_oracle`` for the passage each one follows.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
to something other than itself (printed values of the worked example,
closed forms, textbook library routines, invariants or brute force on tiny
inputs).  No function is "parity unpinned".
"""

from .dlc_oracle import *  # noqa: F401,F403
from .dlc_oracle import __all__  # noqa: F401
