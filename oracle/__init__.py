"""Oracle: a plain, slow, obviously correct CPU implementation of what the
fused dequantize-and-multiply path computes.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything from here.  The
library (``gemm_block_bit_amd``) never imports, links or calls it, and this
package imports nothing from the library: the two share no kernels, headers,
helpers, tables or constants.  Inputs come from ``synth`` (seeded draws only).

Contents
--------
blockquant  group-wise asymmetric RTN over 64x128 blocks of one bitwidth each,
            exact fp32 dequantization, fp64 reference GEMM.
image       an independent reader for the packed block image, written from the
            format description (it never calls the library's packer).
w48         output-feature mixed W8(sym)/W4(asym) x A8(sym) reference: row
            split, weight and activation quantizers, two-step group GEMM.
model       the arithmetic-intensity formula of the MixLLM page.
alloc       offline bitwidth allocation (batched greedy) and bidirectional
            channel reordering, with a weight-magnitude sensitivity proxy.

Precision: quantization decisions for weights are taken in fp64; the
activation quantizer takes them in fp32 (the precision of the GPU kernel
that produces the int8 activations); reference products are fp64.
Every function names the passage it follows.  Functions without an
independent pin say "parity unpinned" -- none currently.
"""
from . import alloc, blockquant, image, model, w48  # noqa: F401
