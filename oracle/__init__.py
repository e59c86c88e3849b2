"""CPU oracle for the int8 Hadamard-domain MoE gate_up path.

This package is TEST INFRASTRUCTURE. It is a plain, slow, fp64 NumPy
implementation of what the GPU library computes, written from the model
cards and independent of the HIP code: the two share no source, no tables,
no helpers. Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import it. The product path never routes through it.

Sources (the pages, by title):
  * "Gemma 4 26B-A4B-it + DFlash, int8 experts — radiance container"
    (called the int8 card below): model table, row "Weights", and the
    section "How this file was made" (the recipe line for the routed
    experts' gate_up tensors).
  * "Gemma 4 26B-A4B-it + DFlash, FP8 experts — radiance container"
    (the FP8 card): model table, row "Weights", and its recipe line.
  * "Gemma 4 12B-it · int8 · for radiance" and "Gemma 4 31B-it · int5 · for
    radiance": header table, row "Format" (per-token, per-128 activation
    scales, the precedent for the FP8 activation quantizer; the 12B card's
    int8 weights + int8 activations are the W8A8 form of w8a8.py).

Modules:
  numfmt   - bf16 and OCP E4M3FN codecs from their bit-level definitions
  hadamard - Sylvester H128, the iterative FWHT, the blockwise rotation
  quant    - int8 RTN with scale search; FP8 128x128 block and per-token
             activation quantizers
  router   - top-k routing, expert histogram, exclusive scan, stable scatter
  gateup   - the grouped gate_up products and the GELU-tanh(gate)*up epilogue
  down     - the bf16 grouped down projection and the weighted combine of a
             token's k expert outputs (the step after the path)
  dense    - the drafter's dense int8 linears with f16 scales (RTN, no
             transform) and their product
  w8a8     - the int8 g128 W8A8 form: RTN weight and per-token activation
             quantizers and the grouped gate_up on integer group sums

Every function here is pinned by tests/test_oracle_*.py against closed
forms, invariants, library special cases or brute force; none is marked
"parity unpinned".
"""

from . import numfmt, hadamard, quant, router, gateup, down, dense, w8a8  # noqa: F401
