"""CPU oracle for block-sparse masked attention (forward and backward).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package's
smoke check and the benchmark's CPU-baseline leg may import, call or execute
anything in this package.  It shares no code with the HIP path and imports
nothing from it; the HIP library never routes through it.

Everything is float64 numpy on the host, written as the plain definition:

* ``masks``     -- the dense boolean visibility mask of one sequence for each
                   mask kind (full, causal, shared-prefix, strip-thinking).
* ``tiles``     -- (BLOCK_M, BLOCK_N) tile classes (empty / partial / full)
                   and the ascending kv-tile index lists, counted from the
                   dense mask.
* ``attention`` -- exact attention by three passes (max, sum of exponentials,
                   normalise) with log-sum-exp, plus a tiled online-softmax
                   variant used only to pin block-size independence.
* ``paged``     -- the gather of a paged KV history through a block table.
* ``forward``   -- drives the above over every sequence and head of a layout.
* ``backward``  -- dQ, dK, dV: the chain rule of the forward map, per
                   sequence and head.

Parity status: every function here is pinned by CPU tests against values the
pages print, closed forms, library special cases, independent constructions
and invariants (see tests/test_oracle_*.py).  No function is unpinned.
"""

from . import masks, tiles, attention, paged, forward, backward  # noqa: F401
