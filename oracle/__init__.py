"""CPU oracle for the grouped block-scaled (MX) GEMM path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
anything in this package: only the tests, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it. It shares
no code, header, table or helper with the HIP library and imports nothing from
it.

What it computes, with the passage each part follows (page titles of the
source pages; no line numbers):

* ``formats``  -- value tables of E2M1, E4M3 (OCP "FN") and UE8M0, built from
  the bit-field definitions of the OCP Microscaling / OCP 8-bit floating point
  specifications. The page "Integrate MXFP4 hipblaslt GEMM support" names
  E2M1 elements with UE8M0 block-32 scales; "route te.GroupedLinear through
  #723; a8w4 fwd-only" names the E4M3 (max 448) activation format.
* ``mx``       -- MX quantization: one UE8M0 scale per 32 elements along the
  contraction axis, shared exponent floor(log2 amax) - emax_elem, clamped to
  [-127, 127], elements rounded to nearest-even and saturated. The tiny-scale
  clamp at -127 and its worked example (amax 2^-126 in E4M3 gives element 2)
  come from the review thread "Clamp tiny block scales to preserve nonzero
  values" on the a8w4 page. Row-wise and segment-padded column-wise layouts
  follow "Triton mxfp4 (and a8w4) grouped GEMM kernel" (the row operand
  (N, K/2) + (N, K/32) and the padded column operand for wgrad).
* ``grouped``  -- grouped forward (TN), input gradient (NN) and variable-K
  weight gradient (NT) on the dequantized operands, contracted in fp64, with
  optional in-place accumulation into an fp32 main_grad ("Add ROCm Triton
  blockwise FP8 grouped GEMM", fused wgrad accumulation).
* ``blockwise`` -- DeepSeek-style blockwise FP8: 1x128 activation scales,
  128x128 weight scales, segment-padded 1x128 column scales, power-of-two
  scales by default, amax floored at 1e-4 ("Add ROCm Triton blockwise FP8
  grouped GEMM").

Parity status: every function is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py``. The non-power-of-two blockwise-FP8 scale mode
(``blockwise.quantize_1x128(..., pow2=False)`` and friends) is our own
reading of a step the page leaves open; its pins are what the arithmetic
fixes (exact power-of-two-amax blocks, the amax element at 448, a half-step
reconstruction bound), which leave open only whether x * q is rounded to
fp32 before encoding.
"""
