"""fp64 CPU oracle for blockwise causal varlen attention.

TEST INFRASTRUCTURE ONLY. This package is the slow, plain reference that the
GPU path is checked against. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import it; the library itself never does,
and it shares no code with the HIP path (no kernels, headers, helpers or
tables). Everything here is numpy in float64.

Parity status of each function is recorded in its docstring. The one function
whose semantics no page pins with a statement or a closed form is the
sliding-window predicate (``window`` in :func:`attention.block_forward`):
"parity unpinned" by the pages; it follows the reading written in its
docstring.
"""

from .attention import *  # noqa: F401,F403
