"""Parity at the full gpt-oss workload sizes, in the launch configuration the bench times, on
every output.

Routing and the CSR are compared whole and bit for bit. Every live output of every stage is
compared with the oracle, which runs one expert at a time (float64 matmul over the decoded
expert): gate_up (act NONE) against the oracle from the same inputs; h (the SwiGLU-OAI
epilogue) within one bf16 ulp of the oracle's activation of the GPU's own g, and within the
carried tolerance of the activation of the oracle's g; down against the oracle fed the GPU's
own h; the combine against the oracle fed the GPU's own d. Padding and ghost rows must keep
the sentinel the outputs were filled with.
"""
import numpy as np
import pytest

import oracle
from mxfp4_mixture_experts_route_amd import _lib as moe
from mxfp4_mixture_experts_route_amd import synth
from helpers import (assert_bf16_within_ulp, assert_swiglu_within, assert_within, bf16_dev,
                     bf16_host, dev, host, live_mask)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

ALPHA, LIMIT = synth.ALPHA, synth.LIMIT
NONE, SWIGLU = moe.MOE_ACT_NONE, moe.MOE_ACT_SWIGLU_OAI
SENT_F32 = 12345.0
SENT_BF16 = 0x4640   # 12288.0

# workload -> projection kernel the bench uses for it (decode_t64 is also checked on the GEMV)
CASES = [("decode_t1", "gemv"), ("decode_t64", "gemm"), ("decode_t64", "gemv"),
         ("prefill_pp512", "gemm"), ("prefill_120b_t2048", "gemm")]


def log(*a):
    print(*a, flush=True)


def sentinel(torch, rows, cols, bf16):
    if bf16:
        return torch.full((rows, cols), SENT_BF16, dtype=torch.int16,
                          device="cuda").view(torch.bfloat16)
    return torch.full((rows, cols), SENT_F32, dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("name,kernel", CASES)
def test_full_size_layer(name, kernel):
    import torch
    wl = synth.WORKLOADS[name]
    log(f"full size {name} via {kernel}: E={wl.E} dim={wl.dim} ffn={wl.ffn} T={wl.T} k={wl.k}")
    tok = synth.tokens(wl, 0)
    W = synth.layer_weights(wl, 0)
    GU = moe.MX4Experts.from_numpy(W["gate_up"])
    DN = moe.MX4Experts.from_numpy(W["down"])
    fn = moe.mx4_moe_gemm if kernel == "gemm" else moe.mx4_moe_gemv

    ids, w = moe.moe_route_topk(dev(tok["logits"]), wl.k)
    ids_ref, w_ref = oracle.route_topk(tok["logits"], wl.k)
    assert np.array_equal(host(ids), ids_ref)
    assert np.array_equal(host(w), w_ref)
    mpad = moe.moe_mpad_max(wl.T, wl.k, wl.E, wl.tile_m)
    counts, basep, row_tok, pos = moe.moe_bucket(ids, wl.E, wl.tile_m, mpad)
    cnt_h, bp_h, rt_h, pos_h = (host(t) for t in (counts, basep, row_tok, pos))
    for nm, g, r in zip(("counts", "basep", "row_tok", "pos"), (cnt_h, bp_h, rt_h, pos_h),
                        oracle.bucket(ids_ref, wl.E, wl.tile_m, mpad)):
        assert np.array_equal(g, r), nm
    live = live_mask(cnt_h, bp_h, mpad)
    x = bf16_dev(tok["x"])
    F, D = wl.ffn, wl.dim

    # gate_up raw (act NONE), every live output
    g = host(fn(x, row_tok, GU, counts, basep, wl.tile_m, mpad, NONE, ALPHA, LIMIT,
                out=sentinel(torch, mpad, 2 * F, False)))
    assert np.all(g[~live] == SENT_F32), "gate_up wrote a padding or ghost row"
    log(f"  oracle gate_up over {int(live.sum())} live rows")
    g_ref, S_g = oracle.project(tok["x"], rt_h, W["gate_up"]["q"], W["gate_up"]["s"],
                                W["gate_up"]["bias"], cnt_h, bp_h, mpad)
    assert_within(g[live], g_ref[live], S_g[live], f"{name} gate_up")

    # h (fused SwiGLU-OAI epilogue): from the GPU's own g within 1 bf16 ulp, and from the
    # oracle's g within the carried tolerance
    h = fn(x, row_tok, GU, counts, basep, wl.tile_m, mpad, SWIGLU, ALPHA, LIMIT,
           out=sentinel(torch, mpad, F, True))
    h_bits = bf16_host(h)
    assert np.all(h_bits[~live] == SENT_BF16), "gate_up + SwiGLU wrote a padding or ghost row"
    assert_bf16_within_ulp(h_bits[live], oracle.bf16_round(oracle.swiglu_oai(g[live], ALPHA,
                                                                             LIMIT)),
                           f"{name} swiglu (GPU g)")
    assert_swiglu_within(h_bits[live], g_ref[live], S_g[live], F, f"{name} swiglu (oracle g)",
                         ALPHA, LIMIT)
    del g, g_ref, S_g

    # down from the GPU's h, every live output
    d = fn(h, None, DN, counts, basep, wl.tile_m, mpad, NONE, ALPHA, LIMIT,
           out=sentinel(torch, mpad, D, False))
    d_h = host(d)
    assert np.all(d_h[~live] == SENT_F32), "down wrote a padding or ghost row"
    log("  oracle down")
    d_ref, d_S = oracle.project(h_bits, None, W["down"]["q"], W["down"]["s"], W["down"]["bias"],
                                cnt_h, bp_h, mpad)
    assert_within(d_h[live], d_ref[live], d_S[live], f"{name} down")
    del d_ref, d_S

    # combine from the GPU's d, every token
    y = host(moe.moe_combine(d, pos, w))
    y_ref, y_S = oracle.combine(d_h, pos_h, w_ref)
    assert_within(y, y_ref, y_S, f"{name} combine")
