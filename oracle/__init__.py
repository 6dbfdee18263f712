"""CPU oracle of the DSA forward path (fp64, numpy).

Test infrastructure, not product code: only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this package.  It shares no
code, headers, tables or helpers with the HIP library and is never called on
the product path.

Parity pins: see the test suite's oracle tests (closed forms, invariants,
exact-rational brute force and library routines).  Nothing here is "parity
unpinned": every function has at least one independent pin.
"""
from . import codecs, dsa  # noqa: F401
