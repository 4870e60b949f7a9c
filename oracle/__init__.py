"""CPU oracle for the quantized paged KV cache -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the HIP
library and its Python binding in ``quantized_paged_kv_kvq_amd``) never imports,
links or calls it, and this package imports nothing from the product path: the
two share no code, constants, tables or helpers.  Both take their inputs from
the seeded generators in ``synth.py``.

What it computes, written plainly and slowly in numpy:

* ``int8_g64``  -- int8 codes with one FP16 scale per 64 values
  (strata PR #2698, section "What it does"; ties-to-even rounding from strata
  PR #120, section "Tests").
* ``q4h``       -- orthonormal Walsh-Hadamard rotation over 256 dims followed by
  q4_0 blocks of 32 (strata PR #2698, section "Not in this PR"; strata PR #120,
  sections "What" and "How").
* ``iso3``      -- IsoQuant 3-bit blocks of 128: L2-normalise, left-multiply each
  4-value group by one unit quaternion, nearest Lloyd-Max centroid, corrected
  norm (FreeToken PR #398, section "What").
* ``paged``     -- page-table addressing of cells and the slab layout.
* ``attention`` -- softmax attention over the dequantised K/V in fp64: decode,
  multi-query verify with per-query causal lengths, and extend over a packed
  prefix plus unquantised new tokens (FreeToken PR #398, section "What").

Precision.  The encoders decide integer codes from floating point, so they
compute in binary32 (the precision the GPU kernels use), one rounding per
operation, no fused multiply-add, correctly rounded division and square root,
round-half-even for ``rint`` and for the binary32 -> binary16 conversion of
scales and norms.  Sums whose order the pages leave open use ``tree_sum`` (a
fixed halving order).  Attention is computed in fp64 from the binary32
dequantised values and rounded once to binary32.

Parity pins.  Every function here is pinned in ``tests/test_oracle_*.py`` by
something other than itself: printed byte counts and ratios, worked examples
of the rounding rules, closed-form error bounds, Hamilton's quaternion rules,
the Lloyd-Max optimality conditions, a library Hadamard matrix, and torch's
scaled-dot-product attention in float64.  Parity unpinned against the pages'
own implementations (their sources and golden vectors are not published):
the ISO3 bit layout, the q4_0 nibble order, and which scale value divides
when codes are made.  Those are pinned only between this oracle and the
kernels.
"""
from . import numerics, int8_g64, q4h, iso3, paged, attention  # noqa: F401
