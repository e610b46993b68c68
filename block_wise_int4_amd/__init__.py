"""MatMulNBits for AMD Instinct MI355X: weight-only block-wise int4 matmul.

The compute path is libmnb.so (HIP kernels for gfx950 behind the C ABI in
include/mnb.h); `block_wise_int4_amd.mnb` is its Python binding.
"""

from .mnb import (  # noqa: F401
    MNB_F16,
    MNB_F32,
    MnbError,
    PackedWeight,
    Plan,
    lib,
    mnb_abi_version,
    mnb_dequant,
    mnb_gemm,
    mnb_gemm_i8,
    mnb_gemm_i8_workspace_bytes,
    mnb_gemm_split_k,
    mnb_gemm_split_k_workspace_bytes,
    mnb_gemm_grouped,
    mnb_gemv,
    mnb_pack,
    mnb_packed_bytes,
    mnb_plan_grouped,
    mnb_quantize_act_i8,
    mnb_quantize_rtn,
    mnb_status_string,
    mnb_unpack,
)
