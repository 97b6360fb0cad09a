"""MI355X-native symmetric int8/int4 group quantization and dequantizing
GEMV/GEMM (HIP kernels for gfx950 behind the C ABI in include/qw.h).

``int8_int4_dequant_amd.qw`` is the binding (loads libqw.so on first use);
``int8_int4_dequant_amd.inputs`` holds the seeded synthetic inputs.
"""
