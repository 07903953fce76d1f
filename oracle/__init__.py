"""Plain float64 CPU reference ("the oracle") of the RMA hot path.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the library and its binding never do, and it
imports nothing from them.  See ``oracle.rma_ref`` for the definitions and the
passages of the pages each one follows.
"""

from .rma_ref import *  # noqa: F401,F403
