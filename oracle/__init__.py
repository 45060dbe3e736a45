"""CPU oracle for the weight-only quantized linear layer.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``bit_weight_only_tq_amd`` and its HIP library) never imports, links or calls
anything here, and nothing here imports the product.  The two share no code:
only the seeded input generators in ``synth`` feed both sides.

What it computes, and where the pages define it
-----------------------------------------------
Sources (three web pages):

* [P1] "Ternary quantized models in vLLM: reverse engineering, reconciliation
  and kernel optimization" (wzjinhao.cn/news/47283).
* [P2] "Model quantization - vLLM runtime quantization architecture"
  (notes.devxops.cn, 2026-05-14).
* [P3] "10.6 Quantization choice and vLLM in practice: decision tree +
  validation" (jennyma11.github.io/infra/ch10-06.html).

Modules:

* ``rne``     - IEEE-754 round-to-nearest-even conversions to binary16 and
                bfloat16, written from the format definitions.
* ``ternary`` - ternary pack / unpack / dequant ([P1] section 1 tip, sections
                3.1-3.2, section 4 naive kernel).
* ``w4``      - W4A16 symmetric int4 pack / unpack / dequant ([P2] sections
                4.2 and 5).
* ``w4asym``  - W4A16 with per-group zero points and activation-order groups
                (g_idx): pack / unpack / dequant ([P2] section 5 (0) and (3)).
* ``gemm``    - fp64 reference product with the dequantized weights and the
                per-element magnitude bound used by the tolerance.
* ``check``   - the tolerance verdict and the ``quant_check`` statistics of
                [P3] section 10.6.3.

Every function comes in a pure-Python loop tier (the specification, for small
inputs) and, where large shapes need it, a numpy tier with the same arithmetic
in the same order.  Floating point is fp64 throughout.  Sums that decide an
integer (the ternary threshold) are sequential in ascending column order; the
numpy tier uses ``cumsum`` (sequential) and never ``sum`` (pairwise).

Readings taken where the pages are silent or garbled are listed in the module
docstrings that use them.  Every function here is pinned by a ``-m "not gpu"``
test against something other than itself (brute force, closed forms, exact
rational arithmetic, library routines, or values the pages print).
"""

from .errors import OracleError  # noqa: F401
