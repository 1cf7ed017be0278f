"""MI355X (gfx950) routed MXFP4 mixture-of-experts chain: HIP kernels behind a C ABI.

The functions below are a thin binding of include/moe_mx4.h (same names); the library is loaded
on first use and must have been built (`python -m mxfp4_mixture_experts_route_amd.build`).
"""
from ._lib import (MOE_ACT_NONE, MOE_ACT_SWIGLU_OAI, MOE_ACT_SWIGLU_OAI_MX8, MX4Experts,
                   MoeError, lib, moe_bucket, moe_combine, moe_layer, moe_mpad_max, moe_route_topk, moe_router,
                   mx4_moe_decode, mx4_moe_decode_persistent,
                   mx4_moe_gemm, mx4_moe_gemm_mx8, mx4_moe_gemv, mx4_pack_experts,
                   mx8_quantize, strerror)

__all__ = ["MOE_ACT_NONE", "MOE_ACT_SWIGLU_OAI", "MOE_ACT_SWIGLU_OAI_MX8", "MX4Experts",
           "MoeError", "lib", "moe_bucket",
           "moe_combine", "moe_layer", "moe_mpad_max", "moe_route_topk", "moe_router",
           "mx4_moe_decode", "mx4_moe_decode_persistent",
           "mx4_moe_gemm", "mx4_moe_gemm_mx8", "mx4_moe_gemv", "mx4_pack_experts",
           "mx8_quantize", "strerror"]
