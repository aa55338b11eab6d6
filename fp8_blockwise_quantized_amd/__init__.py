"""MI355X-native unified-precision FP8 linear layer (Jet-RL quantization flow).

The hot path lives in the HIP library lib/libjetfp8.so behind the C ABI in
include/jetfp8.h; `fp8_blockwise_quantized_amd.jetfp8` is its Python binding
(importing it loads the library and fails if it is not built).
`fp8_blockwise_quantized_amd.inputs` holds the seeded synthetic input
generators and does not need the library.
"""
