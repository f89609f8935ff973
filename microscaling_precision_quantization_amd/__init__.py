"""MI355X-native microscaling quantize + block-scaled GEMM path.

The compute lives in libmxq.so (hand-written HIP for gfx950 behind the C ABI in
include/mxq.h); `binding` is the thin ctypes layer over it, `inputs` holds the
seeded synthetic workloads.
"""

from .binding import (BF16, BF16_NVFP4T, MXFP4, MXFP8, NVFP4, MxqError, abi_version, dequantize, dequantize_transposed,  # noqa: F401
                      gemm_block_scaled, gemm_block_scaled_batch, gemm_fp8_blockwise, gemm_fp8_blockwise_batch, quantize_fp8_block_act, quantize_fp8_block_weight, gemm_mxfp8_matrix_core, grouped_gemm_block_scaled, moe_combine,
                      moe_swiglu_quantize_nvfp4, quantize_mxfp4, quantize_mxfp4_multi, quantize_mxfp8, quantize_mxfp8_multi, quantize_nvfp4,
                      quantize_nvfp4_2d,
                      quantize_nvfp4_per_token, scale_bytes)
