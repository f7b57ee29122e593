"""Plain, slow, obviously correct CPU reference for the Krea 2 joint attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library or its
Python binding) imports, links or calls this package; only the tests, the
``smoke()`` check and the CPU-baseline leg of the benchmark do.  It shares no
code, tables or constants with the HIP path.

Modules:
  plan_ref   -- tile route map (TileMix) and scanline token/block masks
  quant_ref  -- smooth_k mean of K and per-tile symmetric INT8 (float32 emulation)
  attn_ref   -- fp64 attention in the three modes, with optional query slicing

Every function cites the page and section it follows.  The pages are:
  "LayerStream: Krea2 Chunking"              (query slicing, exactness)
  "Krea 2 TileMix Attention (FP16/INT8 tiles)" (dense + tile routing, smooth_k)
  "Krea 2 Scanline Attention"                (scanline block mask)

Parity status: every function here is pinned by the CPU tests in
tests/test_oracle_*.py (brute force, library special cases, closed forms and
invariants).  The positions that the seeded INT8 pick chooses and the reading
of ``tile_aligned`` are fixed by stated readings, not by numbers the pages
print: for those two, parity is unpinned beyond the invariants the tests check.
"""
