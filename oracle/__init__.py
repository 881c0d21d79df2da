"""CPU oracle for batched speculative-sampling verification.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
product path (the HIP library ``libspecv.so`` and its Python binding) never
imports, calls, links or executes it, and this package imports nothing from the
product path.

What is here: a plain, slow, obviously correct implementation of what the hot
path computes, in fp64 numpy, written from the pages' definitions:

* ``philox``   -- the Philox4x32-10 counter-based generator (Salmon, Moraes,
                  Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
                  SC'11) and the stream layout that turns it into uniforms.
* ``sampling`` -- tempered softmax, the accept rule, the residual, the inverse
                  CDF, and chain verification (greedy and sampled).
* ``topf``     -- the SSD/Saguaro bonus-token candidate set (top-F draft logits
                  excluding the drafted token).
* ``tree``     -- SpecInfer's VerifyGreedy and multi-step speculative sampling
                  (MSS) over a token tree.
* ``ssd``      -- Saguaro sampling sigma_{F,C}, per-position fan-out (Theorem
                  12) and the cache-hit check of SSD, and the lenient rule.
* ``ragged``   -- ragged batches (per-sequence draft counts, packed rows) and
                  drafts without probabilities (q = point mass at the token).

Every function cites the page and section it follows. Each is pinned by a
``-m "not gpu"`` test in ``tests/test_oracle_*.py`` against something other
than itself: printed worked examples, closed forms, exact enumeration of the
uniform grid, brute force on tiny inputs, library routines for special cases,
an independent Philox implementation (rocRAND's source header) and the
published Philox known-answer vectors. No function here is "parity unpinned".
"""

from . import philox, ragged, sampling, ssd, topf, tree  # noqa: F401
