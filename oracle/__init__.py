"""CPU oracle for paged grouped-query attention with rotary embeddings.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  The product path (the C-ABI library and its Python binding)
never routes through it and has no CPU fallback.

It is a plain, slow, float64 NumPy restatement of what the AstrAI pages define:

* ``rope``      -- rotary position embedding and its cos/sin table
                   (AstrAI docs/developer/internals.md, "Rotary Position
                   Embedding (RoPE)"; docs/guides/inference.md, "Rotary
                   Embedding Backend"; AstrAI paper, "Model Architecture" table
                   for theta = 10 000).
* ``bf16``      -- round-to-nearest-even rounding to bf16 and the bf16 ulp
                   (AstrAI paper, "BF16 dead zone" paragraph: 7-bit mantissa,
                   ulp 2^-7 at 1.0).
* ``attention`` -- causal mask, decode attention, split-K partials and their
                   log-sum-exp merge, ragged causal prefill over a paged pool
                   (internals.md, "Autoregression & Causal Masking" and "KV
                   Cache Mathematics"; inference.md, "KV Cache", "KVCache
                   System" and "Attention Backend").
* ``pagepool``  -- the page-table builder: contiguous and paged slots, bitmask
                   allocation, reference counts and the exact page-aligned
                   radix prefix cache (inference.md, "KVCache System";
                   internals.md, "Cache Architecture").

It shares no code with the GPU path.  Every function is pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle_*.py`` against facts the pages or
the mathematics fix (the printed 5x5 causal mask, RoPE relative-position
invariance, closed forms, library routines, brute force on tiny inputs).
"""

from . import bf16, rope, attention, pagepool  # noqa: F401
