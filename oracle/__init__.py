"""CPU oracle for NVFP4 weights, 2:4 structured sparsity and the weight-quantised GEMM.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU-baseline leg of
the benchmark may import or run anything in this package. The product path (the HIP
library and its Python binding) never calls it, and this package imports nothing from the
product path; the two share no code. Inputs come from the seeded generators in ``synth``.

Everything here is plain NumPy in float64, slow and written to be checked by eye against
the pages that define the method:

* "NVFP4 Without FP4 Hardware" (ai-muninn.com), section "Convert BF16 to NVFP4 yourself":
  4-bit E2M1 values, one FP8 E4M3 scale per 16 values, one FP32 global scale per tensor;
  section "The shared global scale": a scale may be shared by a group of tensors;
  section "Bit-exact check against lyf's ModelOpt output": decode to BF16 keeping the FP4
  negative zero, re-quantise, compare bytes.
* "NVFP4 vs 2:4 sparse: where the other half of the petaflop went" (robertz.co),
  section "What 2:4 actually is" and its figure: groups of four along the reduction
  dimension, two kept values each carrying a 2-bit position index; section "The byte
  saving is about a quarter, not a half": bits per weight.
* "Sparse GPU FLOPS Need the Right Zeros in the Right Places" (leviathansystems.co),
  section "The operation determines which four entries belong together" (at least two
  zeros per group of four along K) and section "Two half-zero vectors produce different
  pattern answers" (the rule is applied per group, not as a global percentage).

Modules: ``formats`` (E2M1 / E4M3 / bf16 codecs), ``quant`` (NVFP4 quantise/decode),
``sp24`` (2:4 prune, check, compress, decompress), ``gemm`` (fp64 products and the error
bound), ``moe`` (routing, SiLU-gated expert FFN, combine), ``mx`` (MXFP4 quantisation of
activations and weights and the W4A4 product), ``accounting`` (bytes, bits per weight,
roofline and Amdahl arithmetic).

Parity status of each function is stated in its docstring; none is "parity unpinned"
except where said.
"""
from . import formats, quant, sp24, gemm, moe, mx, accounting  # noqa: F401
