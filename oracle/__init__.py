"""CPU oracle for paged attention over a block-paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call,
link or execute anything in this package: only the test suite, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.
It shares no code with the HIP library (no kernels, headers, helpers, tables
or constant generators) and imports nothing from it.

Sources (the three web pages on PagedAttention):
  * "PagedAttention: fragmentation, blocks, block tables" (mlinterviewnotes):
    the block pool, the block table, the slot mapping, copy-on-write, the
    attention metadata and the CPU reference allocator sections.
  * "The pantry of pigeonholes" (blog.lo0.es): "The maths that matter".
  * "Memory management" (llm-inference-explained): "Maths" and "Code".
    Its knobs table and "With KV quantisation" name the FP8 KV cache.

Modules
  sizing      closed forms of the pages' capacity arithmetic
  pool_model  the host block pool (free queue, refcounts, tables, CoW)
  cache_ops   the slot mapping from the block table, the slot scatter and the
              whole-block copy
  attention   fp64 decode and chunked-prefill attention by table gather
  fp8         E4M3 encoding, decoding and per-cache-scale quantisation of
              K/V elements (the FP8 KV cache)

Every floating-point result is computed in fp64 from exact bf16 inputs.
bf16 values travel as uint16 bit patterns (numpy has no bf16 type).

Pins (tests marked ``not gpu``): the numbers the pages print, closed forms,
library routines (torch fp64 scaled_dot_product_attention, scipy logsumexp),
special cases with exact answers, invariances, and a per-token list model
of every sequence for the pool.  No function here is "parity unpinned".
"""
