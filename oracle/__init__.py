"""CPU oracle for the NVFP4 / FP8_DYNAMIC routed-expert MoE path.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that the
HIP library is checked against.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it; the
product path never does, and this package imports nothing from the product
package or its C library.

Every function follows the method as the source pages state it:

* "NVFP4 quantization" page, section "Quantization scheme": weights and input
  activations are 4-bit E2M1 values, each block of 16 values shares one FP8
  E4M3 scale, and each tensor carries one more global scale.
* "FP8 quantization" page, sections "Quantization scheme" and "Quantization
  method": E4M3 weights with a fixed per-output-channel scale, activation
  scales computed per token at run time, weights divided by their scales and
  rounded to the nearest representable FP8 value.
* "Reflection releases Beam" news page, section "Mixture-of-Experts details":
  sigmoid scores over 256 experts, 8 groups of 32, the 4 best groups by the sum
  of each group's two largest scores, top 8 experts inside them, outputs
  combined with normalized router weights and scaled by 2.5; section "Residual
  stream and numerical decisions": router, SwiGLU product and norms in FP32,
  residual weights 1/sqrt(k) and sqrt((k-1)/k).
* "FP8 quantization" page, "Quantization scheme": the attention projections
  and the dense MLPs are FP8_DYNAMIC too (``linear``).
* "NVFP4 quantization" page, "Quantization method": the Local Hessian
  block-scale search of the offline weight quantizer (``hessian``).

Where the pages leave a step open the reading taken is stated in the function
that implements it.  Floating point is evaluated in float64 (exact where the
docstrings say so) and rounded to float32 where the method fixes FP32.

``quant_c`` runs the quantizers of ``quant`` as plain C loops (``quant_c.c``,
built by ``build_c``) for full-size tensors; it is pinned bit-identical to
``quant``.

Parity status of each function (what pins it) is listed in each module header.
"""

from . import formats, quant, route, moe, linear, hessian  # noqa: F401
