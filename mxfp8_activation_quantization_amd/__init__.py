"""MXFP8 o_proj chain for AMD Instinct MI355X (gfx950).

Hand-written HIP kernels behind a C ABI (include/mxfp8.h), bound here with
ctypes; torch supplies device memory and streams.

    mxfp8_quantize      BF16 -> E4M3 codes + packed UE8M0 scales (one per 32 elements)
    mxfp8_rmsnorm_quantize  RMSNorm of BF16 rows, output as MXFP8 (and optionally BF16)
    grouped_fp8_einsum  wo_a: grouped MXFP8 GEMM whose epilogue writes z as MXFP8 and/or BF16
    fp8_gemm_nt         wo_b: MXFP8 GEMM with 1x32 scale blocks on both operands, BF16 out
    o_proj_chain        the chain on one stream (modes: chain, x_fused, unfused)
"""
from .binding import (  # noqa: F401
    CHAIN_MODES,
    MXFP8_ACT_BF16,
    MXFP8_ACT_MXFP8,
    MXFP8ArgumentError,
    MXFP8Error,
    device_check,
    release_retained_workspaces,
    fp8_gemm_nt,
    fp8_gemm_nt_noalloc,
    grouped_fp8_einsum,
    lib,
    mxfp8_quantize,
    mxfp8_rmsnorm_quantize,
    o_proj_chain,
    quantize_weight,
)
