"""Plain, slow, obviously correct CPU oracle for the paged-attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import, call or
link anything under ``oracle/``; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path: no kernels, headers, helpers or constant tables.

Every function cites the passage it follows.  Sources (web pages):

  [IV]  "Inside vLLM: How PagedAttention Changes Python LLM Inference at the
        Systems Level" (ninjatech.agency)
  [RW]  "vLLM PagedAttention: Reducing KV Cache Memory Waste" (cloudai.pt)
  [TG]  "PagedAttention in vLLM: A Throughput Settings Guide" (cloudai.pt)

What the method computes: PagedAttention changes only *where* keys and values
live (fixed-size blocks reached through a per-sequence block table,
[IV §PagedAttention: What the OS Figured Out Decades Ago], [RW §How
PagedAttention Works]); the attention kernel sees the blocks "as if
contiguous".  So the oracle is the plain definition written out: gather each
sequence's blocks into contiguous K/V, then softmax(q K^T * scale) V, all in
float64, output unrounded.

Modules
  attention   gather + dense softmax attention (decode rows, chunked-prefill
              rows), and the partitioned log-sum-exp merge.
  kv_cache    slot-mapped K/V writes and whole-block copies on raw bit
              patterns (bit-exact reference for the write path).
  pool_model  refcounted block pool with copy-on-write.
  splitmix64  the SplitMix64 generator (Steele, Lea, Flood, OOPSLA 2014) used
              to shuffle the pool's initial free list.
  kv_size     the pages' closed form for KV-cache bytes.

Parity pins for every function live in ``tests/test_oracle_*.py``; no function
here is "parity unpinned".
"""
