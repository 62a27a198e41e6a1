"""Reference oracle for the paged KV-cache hot path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package's
``__graft_entry__.smoke()`` check and the CPU-baseline leg of ``bench.py`` may
import anything from here.  The HIP library and its Python binding never do,
and nothing here imports them: the two sides share no code, only the seeded
input generators in ``workloads/``.

What the oracle is
------------------
A plain, slow, obviously correct CPU implementation, in float64, of what the
hot path computes:

* ``metadata``  -- the host-side bookkeeping of a paged cache: block counts,
  the append rule, and the tensors a batch is turned into (slot mapping,
  cumulative sequence lengths, context lengths, padded block tables).
  Source: "3.6 ModelRunner, CUDA Graph, and benchmarks", section 2
  (prepare_prefill / prepare_decode) and section 5 (padding), and the
  "Warmup Guide -- Inference Serving Internals", Chapter 3 (blocks, block
  table, the append off-by-one).
* ``fp8`` -- an 8-bit (OCP E4M3) KV cache: the code of a scaled value
  (round to nearest even, saturating), code values, the quantising store and
  decode over dequantised K/V.  The pages only name a cache-precision flag
  ("10 Serving Engines"); format, rounding and scale are readings, pinned
  against an independent E4M3 implementation (parity partly unpinned by
  the pages).
* ``attention`` -- the slot scatter of new K/V rows, the gather of one
  sequence's K/V through its block table into contiguous arrays, and
  softmax(scale * q K^T) V for decode rows and varlen (chunked) prefill rows
  with a bottom-right causal mask.

Every function states the passage it follows.  Where the pages leave a step
open, the reading taken is stated in the function's docstring.

Pins
----
``tests/test_oracle_*.py`` pin the oracle to things other than itself: the
worked slot-mapping example printed on the ModelRunner page, the block-size
arithmetic of the Warmup Guide, the KV byte counts printed on two pages,
closed forms (one-key context, uniform weights, two-key logistic), the
paged == contiguous and chunked == unchunked invariants, and an independent
pure-Python brute force.  The GQA head mapping (query head h reads KV head
h // G) is a reading the pages do not fix: parity unpinned by the pages for
that one choice; the computation given the mapping is pinned by the
GQA == MHA-with-repeated-heads invariant.
"""

from . import metadata, attention  # noqa: F401
