"""CPU oracle for NVFP4/MXFP4 KV-page quantization and paged FP4 decode attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check of the entry
module and the CPU-baseline leg of the benchmark may import anything here.
The product path (the HIP library and its Python binding) never imports,
calls or falls back to this package, and this package imports nothing from
the product path. The two share no code; the only thing both sides consume is
the seeded synthetic input generator, which holds none of the method's
arithmetic.

It is plain, slow numpy, written from the definitions:

* number formats (``formats``): FP4 E2M1 element codes, FP8 E4M3 and E8M0
  block scales, from the OCP 8-bit Floating Point and OCP Microscaling (MX)
  v1.0 specifications;
* the 128-point Hadamard rotation (``rotation``);
* block quantizers ``amax6``, ``four_six``, ``mxfp4_search`` and the
  underflow-aware ``amax2_or_amax6`` probability quantizer (``quant``);
* the physical page layout of the quantized cache (``layout``);
* the page writer (``writer``) and decode attention in float64 over the
  quantized operands with an explicit partition plan (``decode``);
* recipe defaults and validation (``recipe``).

The method's names and constants come from three web pages:
"BitDecoding-FP4 evaluation/config.py" (OpenBitSys/BitDecoding-FP4),
"kv-landlords scripts/quant_ab.py" and the gitdiagram summary
"How openbitsys/bitdecoding-fp4 works". The pages give names, constants and
validation rules but no formulas; where they leave a step open the oracle
takes one plain reading and says so in the function that implements it.
Functions whose rule is such a reading (the four_six and mxfp4_search
criteria, the amax2_or_amax6 branch, the sink partition, the P normaliser
and the float32 form of p', and the block shape of the channel key scale
geometry) are pinned only by
invariants and brute force, not by values printed on the pages: their parity
is "parity unpinned" with respect to the pages' own implementation.
"""
