"""Plain fp64 CPU oracle for KV-parallel (sequence-split) decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library (no kernels, headers, helpers, tables or
constant generators) and it never imports the library's binding.

Sources (the web pages about Helix Parallelism that define the method):

* "Helix Parallelism: Rethinking Sharding Strategies for Interactive
  Multi-Million-Token LLM Decoding" (fdeinterviews.com paper summary),
  paragraph on KV parallelism: every KV slice attends over its part of the
  history and returns a partial output and a log-sum-exp; one exchange
  combines them into the exact result.  Same page, paragraph on Helix's two
  layouts: new KV entries rotate over the KV-parallel ranks every 16 tokens.
* jaehun.me paper review, Prompt 1.3.2 "The Secret Weapon": the boxed
  LSE-weighted rescaling formula for the partial outputs, stated to be exact.
* open-lab.net (NVIDIA technical blog, Korean), section on distributed KV
  placement: with two KV-parallel ranks, tokens 1-16 go to rank 0 and tokens
  17-32 to rank 1.
* ifai.io news article on NVIDIA's Helix, section "Decoupling attention and
  FFN".

The modules cite these pages as "Helix summary", "jaehun.me review", "NVIDIA
blog" and "ifai.io article".

Modules
-------
placement   token -> (slice, local row) map and slice lengths
codecs      fp8 e4m3, e2m1 (fp4) and e8m0 decoding from the bit definitions
attention   unsplit softmax attention, per-slice partials, LSE combine

Parity status: every function here is pinned by tests in
``tests/test_oracle_pins.py`` (brute force, closed forms, invariants, the
pages' placement example, published format specs).  No function is "parity
unpinned".
"""

from . import attention, codecs, placement  # noqa: F401
