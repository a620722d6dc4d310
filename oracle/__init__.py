"""CPU oracle for the NVFP4 / FP8_DYNAMIC routed-expert MoE path.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that the
HIP library is checked against.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it; the
product path never does, and this package imports nothing from the product
package or its C library.

Every function follows the method as the source pages state it:

* "NVFP4 quantization" page, section "Quantization scheme": expert weights
  and expert inputs are held as 4-bit E2M1 codes; every run of 16 values has
  its own FP8 E4M3 scale, and the tensor one FP32 scale on top of those.
* "FP8 quantization" page, sections "Quantization scheme" and "Quantization
  method": E4M3 codes; a weight row (output channel) has one fixed scale, an
  activation row (token) one scale found at run time; a value is divided by
  its scale and the quotient becomes the closest E4M3 value (RTN).
* "Reflection releases Beam" news page, section "Mixture-of-Experts details":
  each of the 256 experts gets a sigmoid score; of the 8 groups of 32 experts
  the 4 whose two highest scores add up to the most survive; the 8
  highest-scoring experts of those are chosen, and their outputs are mixed
  with the chosen scores renormalized to sum to one, the total times 2.5;
  section "Residual stream and numerical decisions": router, SwiGLU product
  and norms in FP32, residual weights 1/sqrt(k) and sqrt((k-1)/k).
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
