"""KDA oracle package: TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct CPU references for the KDA hot path. Only the
test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything from here; the product path (the HIP library
and its Python binding) never does, and shares no code with it.

Modules:
  oracle.reference  -- ctypes front end of the C fp64 token-by-token oracle
  oracle.brute      -- exact rational recurrence and dense transition products
  oracle.chunk_spec -- fp64 chunked (matmul) form, used to pin chunk algebra
  oracle.frontend   -- fp64 front end: q/k L2 normalisation, gate and beta
                       from raw logits
  oracle.variants   -- GDN (one decay per head) and DeltaNet (no decay) gates
                       as per-channel KDA gates
"""
