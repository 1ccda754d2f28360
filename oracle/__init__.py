"""CPU oracle for the W4A16 and W8A8-FP8 quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import anything from this package.  The
product path (the HIP library and its Python binding) never calls it and
shares no code with it: no kernels, headers, helpers, tables or constants.

Everything here is plain, slow and written to be checked against the pages by
eye: numpy float32 where the method fixes fp32 (scale division, dequantized
weights), float64 for the matrix products.

Modules
-------
bf16          round-to-nearest-even fp32 -> bf16 and back.
int4_g128     symmetric INT4 RTN quantization in 128-row groups with a zero
              offset of 8, the canonical and the native (MFMA fragment order)
              packings, unpacking, dequantization and the W4A16 product.
fp8_e4m3      the OCP e4m3fn codec, per-output-channel weight quantization,
              dynamic per-token activation quantization, the native weight
              order and the W8A8-FP8 product.
decode_model  the two-term decode-step model (memory pipe vs math pipe).
mse_clip      MSE-optimal clipping of the INT4 group scale by grid search.

Parity unpinned (nothing outside the oracle fixes these): the native byte
orders beyond their own written specification.
"""
