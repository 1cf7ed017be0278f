"""Parity at the full gpt-oss workload sizes, in the launch configuration the bench times.

Routing and the CSR are compared whole and bit for bit. The projections are too large for the
CPU oracle in full, so each stage is checked on sampled outputs (rows, columns) that the oracle
evaluates one by one from the GPU stage's own inputs; the combine is checked on sampled tokens.
"""
import numpy as np
import pytest

import oracle
from mxfp4_mixture_experts_route_amd import _lib as moe
from mxfp4_mixture_experts_route_amd import synth
from helpers import (assert_bf16_within_ulp, assert_within, bf16_dev, bf16_host, dev, host,
                     live_mask)

pytestmark = pytest.mark.gpu

ALPHA, LIMIT = synth.ALPHA, synth.LIMIT
NONE, SWIGLU = moe.MOE_ACT_NONE, moe.MOE_ACT_SWIGLU_OAI
N_SAMPLES = 256

# workload -> projection kernel the bench uses for it (decode_t64 is also checked on the GEMV)
CASES = [("decode_t1", "gemv"), ("decode_t64", "gemm"), ("decode_t64", "gemv"),
         ("prefill_pp512", "gemm"), ("prefill_120b_t2048", "gemm")]


def log(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("name,kernel", CASES)
def test_full_size_layer(name, kernel):
    wl = synth.WORKLOADS[name]
    rng = np.random.default_rng(17)
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
    live_rows = np.flatnonzero(live_mask(cnt_h, bp_h, mpad))
    x = bf16_dev(tok["x"])

    # gate_up raw on sampled (row, n)
    g = host(fn(x, row_tok, GU, counts, basep, wl.tile_m, mpad, NONE, ALPHA, LIMIT))
    rows = rng.choice(live_rows, N_SAMPLES)
    cols = rng.integers(0, 2 * wl.ffn, N_SAMPLES)
    ref, S = oracle.project_at(tok["x"], rt_h, W["gate_up"]["q"], W["gate_up"]["s"],
                               W["gate_up"]["bias"], cnt_h, bp_h, list(zip(rows, cols)))
    assert_within(g[rows, cols], ref, S, f"{name} gate_up")

    # SwiGLU from the GPU's own g, on sampled (row, j)
    h = fn(x, row_tok, GU, counts, basep, wl.tile_m, mpad, SWIGLU, ALPHA, LIMIT)
    h_bits = bf16_host(h)
    js = rng.integers(0, wl.ffn, N_SAMPLES)
    pair = np.stack([g[rows, js], g[rows, wl.ffn + js]], axis=1)
    assert_bf16_within_ulp(h_bits[rows, js],
                           oracle.bf16_round(oracle.swiglu_oai(pair, ALPHA, LIMIT)[:, 0]),
                           f"{name} swiglu")

    # down from the GPU's h on sampled (row, n)
    d = fn(h, None, DN, counts, basep, wl.tile_m, mpad, NONE, ALPHA, LIMIT)
    d_h = host(d)
    dcols = rng.integers(0, wl.dim, N_SAMPLES)
    ref, S = oracle.project_at(h_bits, None, W["down"]["q"], W["down"]["s"], W["down"]["bias"],
                               cnt_h, bp_h, list(zip(rows, dcols)))
    assert_within(d_h[rows, dcols], ref, S, f"{name} down")

    # combine from the GPU's d on sampled tokens (all columns)
    y = host(moe.moe_combine(d, pos, w))
    toks = np.unique(rng.integers(0, wl.T, min(16, wl.T)))
    y_ref, y_S = oracle.combine(d_h, pos_h[toks], w_ref[toks])
    assert_within(y[toks], y_ref, y_S, f"{name} combine")
