"""CPU float64 oracle for PISA block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only the test-suite, the package's smoke check and the
benchmark's CPU-baseline leg do.  It shares no code with the HIP library.

Modules:
  pisa_oracle  vectorised NumPy float64 definition (stats, selection, attention)
  bruteforce   scalar Python-loop re-statement of the same definition, with
               exact rational ranking, for tiny inputs only

Parity pins: every function here is pinned by tests marked ``not gpu``
(closed forms, the sliding-window page's worked example, special cases that
reduce to dense softmax attention, convergence orders, brute force).  No
function is "parity unpinned".
"""
from . import pisa_oracle  # noqa: F401
