"""CPU oracle of the routed MXFP4 expert chain — test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
It shares no code with the HIP library and never imports it.
"""
from .mx4_oracle import (E2M1_TABLE, E4M3_MAX, FP32_OVERFLOW, bf16_round, bf16_to_f64, bucket,
                         chain, chain_mx8, combine, dequant, dequant_exact, e2m1_decode,
                         e4m3_decode, e4m3_encode, e8m0_decode, live_rows, mpad_max,
                         mx8_dequant, mx8_quantize, project, project_at, project_mx8,
                         project_mx8_at, project_values, round_fp32_range, route_topk,
                         router_logits, swiglu_oai, unpack_codes)

__all__ = ["E2M1_TABLE", "E4M3_MAX", "FP32_OVERFLOW", "bf16_round", "bf16_to_f64", "bucket",
           "chain", "chain_mx8", "combine", "dequant", "dequant_exact", "e2m1_decode",
           "e4m3_decode", "e4m3_encode", "e8m0_decode", "live_rows", "mpad_max", "mx8_dequant",
           "mx8_quantize", "project", "project_at", "project_mx8", "project_mx8_at",
           "project_values", "round_fp32_range", "route_topk", "router_logits", "swiglu_oai",
           "unpack_codes"]
