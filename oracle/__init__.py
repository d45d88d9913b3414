"""CPU oracle for the MXFP8 block-scaled top-k MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (the HIP library and its Python binding) never imports, calls or links it,
and it never imports the product path: the two share no code, tables or
constants.

The oracle is plain NumPy in float64, written to be read against the pages that
define the method:

* "Quantization on Ascend" (sglang docs), section on MXFP8 for LLM MoE models:
  e4m3 payload, e8m0 scale stored as exponent + 127, block of 32 along the
  reduction dimension, scale reshaped from [N, K/32] to [N, K/64, 2] by
  contiguous pairing; the forward is routing with fused activation quant, then
  grouped GEMM1 fused with SwiGLU and requantisation, then grouped GEMM2.
* "[WIP] Fix offline W8A8 MXFP8 quantization for Qwen3.5 on Ascend NPU"
  (sglang PR 32266), commit that adds the fused-experts chain (routing, act
  quant, swiglu-quant GEMM, grouped GEMM, finalize routing) and the Summary
  paragraph on the offline partial MXFP8 block-scale layout (ceil(K/32)
  scales, odd count padded with one zero partner).
* "PR #30768 report" (prhub), key source excerpt: GEMM1 takes a cumulative
  group list, the dispatcher produces counts.

Modules:
  mx_ref   -- e4m3 / e8m0 / bf16 codecs, MX block quantise / dequantise
  moe_ref  -- routing, grouped GEMMs, SwiGLU + requant, finalize, the whole
              layer, a per-token brute-force dense MoE, and the top-k
              softmax router upstream of the layer

Every function states which passage it follows, or which reading of a silent
passage it takes (the readings are listed in the design notes).
"""

from . import mx_ref  # noqa: F401
