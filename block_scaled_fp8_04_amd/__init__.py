"""Block-scaled FP8 linear path for AMD Instinct MI355X (gfx950).

The library is ``libbfp8.so`` (hand-written HIP, C ABI in ``include/bfp8.h``);
``block_scaled_fp8_04_amd._lib`` is its thin Python binding.  Importing the
package does not load the library; the first call does, and raises if it has
not been built (``__graft_entry__.build()``).
"""
from ._lib import (  # noqa: F401
    BLOCK, Bfp8Error, EXPORTS, LIBRARY, act_quant, bfp8_act_quant, bfp8_bf16_round_range,
    bfp8_e4m3_encode_range,
    bfp8_gemm, bfp8_gemm_grouped, bfp8_gemm_kernel_name, bfp8_gemm_workspace_size, bfp8_status_string, bfp8_version,
    bfp8_weight_dequant, gemm, gemm_grouped, library, linear_fp8, status_string, weight_dequant,
    bfp8_act_quant_rows, bfp8_moe_combine, bfp8_moe_dispatch, bfp8_moe_dispatch_workspace_size,
    moe_combine, moe_dispatch, moe_experts_fp8, bfp8_gemm_bf16, bfp8_gemm_bf16_workspace_size,
    gemm_bf16, linear_bf16,
    bfp8_gemm_act_quant, gemm_act_quant, bfp8_gemm_swiglu_act_quant, gemm_swiglu_act_quant,
    interleave_w13, bfp8_act_quant_ue8m0, bfp8_gemm_ue8m0, bfp8_gemm_ue8m0_workspace_size, act_quant_ue8m0,
    gemm_ue8m0,
    bfp8_linear_fp8, bfp8_linear_fp8_workspace_size, linear_workspace, bfp8_gemm_noalloc,
    NOALLOC_SCRATCH_BYTES,
)
