"""CPU oracle for rotate-then-quantize KV-cache compression and decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in this
package.  The product path (the HIP library and its Python binding) never routes
through it, and shares no code, tables or constants with it.

What it computes, in the order the pages give it:

* ``rotation``  -- the random sign flip followed by a Walsh-Hadamard transform
  (the Hadamard form of the randomized rotation in "When Quantization Is Free",
  Methodology section 1), or a fixed dense orthogonal matrix ("OSCAR", section
  2.2A, composite rotation).  The write side is emulated bit-exactly in fp32;
  the query/output rotations are done in fp64.
* ``numerics``  -- fp16/bf16 rounding, the OCP E4M3 and E2M1 value tables built
  by enumerating every bit pattern, and round-half-to-even of exact quotients.
* ``codec``     -- per-group scales (absmax, clipped, searched), codes, the
  packed byte layout of the cache, and the inverse (unpack/dequantize).
* ``attention`` -- single-token decode attention in fp64 over the decoded cache,
  with optional exact recompute of flagged blocks from fp16 originals.
* ``bound``     -- per-block error descriptors, the certified per-block bound
  and the output certificate ("Runtime-Certified Bounded-Error Quantized
  Attention", Methodology section 2).
* ``adaptive``  -- the adaptive-precision steps of the same page (Methodology
  section 3): block attention mass estimated from the quantized keys, the
  top-K* blocks covering a mass fraction, and the dense fallback of a head.

Every function names the passage it follows in its docstring.  Where a page is
silent, the reading taken is stated there.
"""

from . import numerics, rotation, codec, attention, bound, adaptive  # noqa: F401

__all__ = ["numerics", "rotation", "codec", "attention", "bound"]
