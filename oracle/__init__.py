"""CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code with the HIP library (``paged_kv_cache_263_amd``) and imports
nothing from it.

Contents (each function cites the passage of the source pages it follows):

* ``oracle.pool``      - block pool, free list, refcounts, per-sequence block
                         tables, sharing and copy-on-write, plus a host byte
                         store that writes and reads tokens through the tables.
* ``oracle.fp8``       - the OCP E4M3 (fp8) format written out from its
                         definition: decode of all 256 codes, round-to-nearest-
                         even quantisation with saturation.
* ``oracle.int8``      - the symmetric INT8 storage (code * scale, round half to
                         even, clamped to +-127) written out from its definition.
* ``oracle.attention`` - softmax(q K^T / sqrt(d)) V in float64 for a decode
                         query and for a causal prefill chunk, with grouped-
                         query head sharing.

Pages cited (by title and section):

* [P1] "PagedAttention, chunked prefill, and the launch that cascades"
  (deepnotes.pages.dev).
* [P2] "Waste, and three ways to reclaim it" (runbooks.in, LLM Inference
  Runbook, document 10).
* [P3] "M.65 Inference Serving" (systemdesigntutorial.com).

Every function in this package is pinned by tests under ``tests/`` marked
``not gpu`` (closed forms, invariants stated on the pages, library routines
for special cases, hand-worked fixtures under ``tests/golden/``).
"""

from . import attention, fp8, int8, pool  # noqa: F401
