"""Parity of the MXFP8-activation variant (mx8_quantize, mx4_moe_gemm_mx8) with the oracle,
through the C ABI.

Protocol: quantized activations (E4M3 bytes and e8m0 scales, padding included) are compared
bit for bit, since both sides take every rounding decision on exact values. Each projection is
compared with oracle.project_mx8 fed the GPU's own quantized rows, per element within
|gpu - ref| <= 1e-3 * S + 1e-5 (S = |bias| + sum |x_i w_i|), the SwiGLU output within one bf16
ulp of the oracle's activation of the GPU's own fp32 result; exact-arithmetic cases and the
one-hot MXFP4 decode sweep must match exactly.
"""
import numpy as np
import pytest

import oracle
from mxfp4_mixture_experts_route_amd import _lib as moe
from mxfp4_mixture_experts_route_amd import synth
from helpers import (assert_bf16_within_ulp, assert_equal_values, assert_swiglu_within,
                     assert_within, bf16_dev,
                     bf16_host, dev, host, live_mask)
from test_gpu_parity import EDGE, MEDIUM, SENT_BF16, SENT_F32, case, front, sentinel_out

pytestmark = pytest.mark.gpu

ALPHA, LIMIT = synth.ALPHA, synth.LIMIT
NONE, SWIGLU = moe.MOE_ACT_NONE, moe.MOE_ACT_SWIGLU_OAI


def log(*a):
    print(*a, flush=True)


def quant_gpu(bits, live=None):
    q, s = moe.mx8_quantize(bf16_dev(bits), None if live is None else dev(live.astype(np.int32)))
    return host(q), host(s)


def assert_quant_equal(q, s, bits, what):
    """GPU MXFP8 rows (q [rows][K], s [rows][SP]) equal the oracle's, padding bytes zero."""
    K = bits.shape[1]
    KB = K // 32
    q_ref, s_ref = oracle.mx8_quantize(bits)
    bad = np.argwhere(q != q_ref)
    assert len(bad) == 0, f"{what}: {len(bad)} codes differ; first at {tuple(bad[0])}: " \
        f"gpu={q[tuple(bad[0])]:#x} ref={q_ref[tuple(bad[0])]:#x}"
    assert np.array_equal(s[:, :KB], s_ref), f"{what}: scales differ"
    assert not s[:, KB:].any(), f"{what}: scale padding not zero"


def crafted_rows(seed, rows, K):
    """bf16 rows with the hard cases of the conversion: magnitudes across the bf16 range,
    subnormals, zeros of both signs, exact ties between E4M3 neighbours, saturation."""
    g = np.random.default_rng(seed)
    v = g.standard_normal((rows, K)) * np.exp2(g.integers(-60, 60, (rows, 1)))
    mags = oracle.e4m3_decode(np.arange(127))
    mids = (mags[:-1] + mags[1:]) / 2                      # ties once scaled by the block max
    for r in range(0, rows, 4):
        blk = g.choice(mids, K) * g.choice([-1.0, 1.0], K)
        blk[::32] = 448.0 * g.choice([1.0, 1.0625, 1.125], K // 32)   # pins X; some saturate
        v[r] = blk * np.exp2(float(g.integers(-100, 100)))
    v[1 % rows, :32] = 0.0
    v[1 % rows, 1:32:2] = -0.0
    v[2 % rows, 32 % K:64 % K or K] = g.standard_normal(32 if K >= 64 else K) * 2.0 ** -130
    v[3 % rows, :] = np.clip(v[3 % rows, :] * 1e38, -3.38e38, 3.38e38)
    return oracle.bf16_round(v)


@pytest.mark.parametrize("rows,K", [(1, 32), (7, 96), (33, 2880), (5, 4128), (300, 64)])
def test_quantize_bit_exact(rows, K):
    log(f"mx8_quantize rows={rows} K={K}")
    bits = crafted_rows(rows * 131 + K, rows, K)
    q, s = quant_gpu(bits)
    assert_quant_equal(q, s, bits, f"quantize {rows}x{K}")


def test_quantize_skips_rows_that_are_not_live():
    import torch
    rows, K = 40, 160
    bits = crafted_rows(5, rows, K)
    live = np.where(np.arange(rows) % 3 == 1, -1, np.arange(rows)).astype(np.int32)
    q = torch.full((rows, K), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((rows, 16), 0xCD, dtype=torch.uint8, device="cuda")
    moe.mx8_quantize(bf16_dev(bits), dev(live), out=(q, s))
    q, s = host(q), host(s)
    on = live >= 0
    assert np.all(q[~on] == 0xAB) and np.all(s[~on] == 0xCD)
    assert_quant_equal(q[on], s[on], bits[on], "live rows")


def gemm8(aq, as_, a_row, W, counts, basep, tile_m, mpad, act, out=None):
    if act == moe.MOE_ACT_SWIGLU_OAI_MX8:
        q, s = out if out is not None else (None, None)
        return moe.mx4_moe_gemm_mx8(aq, as_, a_row, W, counts, basep, tile_m, mpad, act, ALPHA,
                                    LIMIT, out=q, out_scale=s)
    return moe.mx4_moe_gemm_mx8(aq, as_, a_row, W, counts, basep, tile_m, mpad, act, ALPHA, LIMIT,
                                out=out)


def staged_mx8(c):
    """The chain on MXFP8 activations, each stage checked against the oracle fed the GPU's own
    previous-stage output."""
    E, D, F, tile_m = c["E"], c["D"], c["F"], c["tile_m"]
    mpad, (counts, basep, row_tok, pos), (cnt_h, bp_h, rt_h, pos_h) = front(c["ids"], E, tile_m)
    live = live_mask(cnt_h, bp_h, mpad)
    GU = moe.MX4Experts.from_numpy(c["gu"])
    DN = moe.MX4Experts.from_numpy(c["dn"])

    xq, xs = moe.mx8_quantize(bf16_dev(c["x"]))
    xq_h, xs_h = host(xq), host(xs)
    assert_quant_equal(xq_h, xs_h, c["x"], "x")
    KB = D // 32

    g = host(gemm8(xq, xs, row_tok, GU, counts, basep, tile_m, mpad, NONE,
                   out=sentinel_out(mpad, 2 * F, NONE)))
    g_ref, g_S = oracle.project_mx8(xq_h, xs_h[:, :KB], rt_h, c["gu"]["q"], c["gu"]["s"],
                                    c["gu"]["bias"], cnt_h, bp_h, mpad)
    assert_within(g[live], g_ref[live], g_S[live], "gate_up mx8")
    assert np.all(g[~live] == SENT_F32)

    h = gemm8(xq, xs, row_tok, GU, counts, basep, tile_m, mpad, SWIGLU,
              out=sentinel_out(mpad, 2 * F, SWIGLU))
    h_bits = bf16_host(h)
    assert_bf16_within_ulp(h_bits[live], oracle.bf16_round(oracle.swiglu_oai(g[live], ALPHA, LIMIT)),
                           "swiglu mx8")
    assert np.all(h_bits[~live] == SENT_BF16)

    hq, hs = moe.mx8_quantize(h, live=row_tok)
    hq_h, hs_h = host(hq), host(hs)
    assert_quant_equal(hq_h[live], hs_h[live], h_bits[live], "h")

    # the fused epilogue writes the same MXFP8 rows (h rounded to bf16 in-register, then the
    # same conversion); rows that are not live stay untouched
    if F % 32 == 0:
        import torch
        q2 = torch.full((mpad, F), 0xAB, dtype=torch.uint8, device="cuda")
        s2 = torch.full((mpad, moe.scale_row_bytes(F)), 0xCD, dtype=torch.uint8, device="cuda")
        gemm8(xq, xs, row_tok, GU, counts, basep, tile_m, mpad, moe.MOE_ACT_SWIGLU_OAI_MX8,
              out=(q2, s2))
        q2h, s2h = host(q2), host(s2)
        assert np.array_equal(q2h[live], hq_h[live]) and np.array_equal(s2h[live], hs_h[live]), \
            "fused MXFP8 h"
        assert np.all(q2h[~live] == 0xAB) and np.all(s2h[~live] == 0xCD)

    d = host(gemm8(hq, hs, None, DN, counts, basep, tile_m, mpad, NONE,
                   out=sentinel_out(mpad, D, NONE)))
    with np.errstate(invalid="ignore", over="ignore"):   # rows that are not live hold garbage
        d_ref, d_S = oracle.project_mx8(hq_h, hs_h[:, :F // 32], None, c["dn"]["q"], c["dn"]["s"],
                                        c["dn"]["bias"], cnt_h, bp_h, mpad)
    assert_within(d[live], d_ref[live], d_S[live], "down mx8")
    assert np.all(d[~live] == SENT_F32)
    return mpad, d, (counts, basep, row_tok, pos), (cnt_h, bp_h, rt_h, pos_h)


def test_staged_chain_medium_mx8():
    c = case(**MEDIUM)
    log(f"staged chain mx8: E={c['E']} D={c['D']} F={c['F']} T={c['T']} k={c['k']}")
    staged_mx8(c)


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases_mx8(name):
    c = case(**EDGE[name])
    log(f"edge mx8 {name}: E={c['E']} D={c['D']} F={c['F']} T={c['T']} k={c['k']} "
        f"tile_m={c['tile_m']}")
    staged_mx8(c)


def test_layer_mx8_matches_oracle_chain():
    # moe_layer(projection="gemm_mx8") end to end against oracle.chain_mx8 from inputs only:
    # routing, CSR and quantized x bit for bit; y within the chain tolerance (h may flip one
    # bf16 rounding, which can move a quantized h element by one E4M3 step)
    c = case(**MEDIUM)
    log("layer mx8 vs oracle.chain_mx8")
    out = moe.moe_layer(bf16_dev(c["x"]), dev(c["logits"]), moe.MX4Experts.from_numpy(c["gu"]),
                        moe.MX4Experts.from_numpy(c["dn"]), c["k"], c["tile_m"], ALPHA, LIMIT,
                        projection="gemm_mx8")
    ref = oracle.chain_mx8(c["x"], c["logits"], c["gu"], c["dn"], c["k"], c["tile_m"], ALPHA,
                           LIMIT)
    for key in ("ids", "counts", "basep", "row_tok", "pos", "xq"):
        assert np.array_equal(host(out[key]), ref[key]), key
    assert np.array_equal(host(out["xs"])[:, :c["D"] // 32], ref["xs"])
    assert np.array_equal(host(out["w"]), ref["w"])
    assert_within(host(out["y"]), ref["y"], ref["y_S"], "chain mx8 end-to-end", rel=5e-2)


def test_exact_arithmetic_mx8():
    # small integers quantize exactly (block max 4 -> scale 2^-6, every value a multiple of 64)
    # and every partial sum is exact, so GPU == oracle exactly
    g = np.random.default_rng(3)
    E, D, F, T, k, tile_m = 5, 160, 96, 40, 3, 16
    x = synth.round_f32_to_bf16_bits(g.integers(-4, 5, (T, D)).astype(np.float32))
    x[:, ::32] = synth.round_f32_to_bf16_bits(np.full((T, D // 32), 4.0, np.float32))
    gu = {"q": g.integers(0, 256, (E, 2 * F, D // 2)).astype(np.uint8),
          "s": g.integers(126, 128, (E, 2 * F, D // 32)).astype(np.uint8),
          "bias": (g.integers(-8, 9, (E, 2 * F)) / 4).astype(np.float32)}
    ids = synth.random_ids(9, T, k, E)
    log("exact arithmetic mx8")
    mpad, (counts, basep, row_tok, _), (cnt_h, bp_h, rt_h, _) = front(ids, E, tile_m)
    live = live_mask(cnt_h, bp_h, mpad)
    xq, xs = moe.mx8_quantize(bf16_dev(x))
    assert np.array_equal(oracle.mx8_dequant(host(xq), host(xs)[:, :D // 32]),
                          oracle.bf16_to_f64(x))
    out = host(gemm8(xq, xs, row_tok, moe.MX4Experts.from_numpy(gu), counts, basep, tile_m,
                     mpad, NONE))
    ref, _ = oracle.project(x, rt_h, gu["q"], gu["s"], gu["bias"], cnt_h, bp_h, mpad)
    assert_equal_values(out[live], ref[live], "gate_up exact mx8")


def test_one_hot_decode_sweep_mx8():
    # every (e2m1 code, e8m0 scale) weight pair times a one-hot activation of 1.0 (E4M3 256 at
    # scale 2^-8) through the MX-scaled MFMA: the output is the decoded weight itself
    K = 32
    N = 2 * 16 * 256
    q = np.zeros((1, N, K // 2), dtype=np.uint8)
    s = np.zeros((1, N, 1), dtype=np.uint8)
    for half in range(2):
        for code in range(16):
            for e in range(256):
                n = half * 4096 + code * 256 + e
                if half == 0:
                    q[0, n, 0] = code
                else:
                    q[0, n, 15] = code << 4
                s[0, n, 0] = e
    x = np.zeros((2, K), dtype=np.float32)
    x[0, 0] = 1.0
    x[1, 31] = 1.0
    xb = synth.round_f32_to_bf16_bits(x)
    ids = np.zeros((2, 1), dtype=np.int32)
    log("one-hot sweep mx8")
    mpad, (counts, basep, row_tok, _), (cnt_h, bp_h, rt_h, _) = front(ids, 1, 1)
    xq, xs = moe.mx8_quantize(bf16_dev(xb))
    W = {"q": q, "s": s, "bias": None}
    out = host(gemm8(xq, xs, row_tok, moe.MX4Experts.from_numpy(W), counts, basep, 1, mpad,
                     NONE))[:2]
    with np.errstate(invalid="ignore", over="ignore"):
        ref, _ = oracle.project_mx8(host(xq), host(xs)[:, :1], rt_h, q, s, None, cnt_h, bp_h,
                                    mpad)
    # all 256 scale bytes: the activated weight comes out decoded (infinite beyond the fp32
    # range, NaN for byte 255); the MX dot product scales each block's exact sum, so the zero
    # activation times a weight beyond the fp32 range gives 0 (in the oracle too), every output
    # compared
    ref = ref[:2]
    scale = np.tile(np.arange(256), 32)
    assert np.all(np.isnan(ref) == (scale == 255)[None, :])
    assert np.isinf(ref).sum() == 24 and np.all(ref[np.isinf(out)] == out[np.isinf(out)])
    assert_equal_values(out, ref, "one-hot decode mx8")


@pytest.mark.parametrize("N,K,act", [(40, 64, NONE), (36, 64, SWIGLU), (264, 96, NONE),
                                     (2 * 130, 64, SWIGLU), (8, 32, NONE), (400, 4096, NONE)])
def test_projection_ragged_n_mx8(N, K, act):
    E, T, k, tile_m = 3, 25, 2, 16
    W = synth.random_mx4(N + K, E, N, K)
    xb = synth.random_bf16(N, (T, K))
    ids = synth.random_ids(N, T, k, E)
    log(f"ragged mx8 N={N} K={K} act={act}")
    mpad, (counts, basep, row_tok, _), (cnt_h, bp_h, rt_h, _) = front(ids, E, tile_m)
    live = live_mask(cnt_h, bp_h, mpad)
    Wd = moe.MX4Experts.from_numpy(W)
    xq, xs = moe.mx8_quantize(bf16_dev(xb))
    xq_h, xs_h = host(xq), host(xs)[:, :K // 32]
    g = host(gemm8(xq, xs, row_tok, Wd, counts, basep, tile_m, mpad, NONE))
    g_ref, g_S = oracle.project_mx8(xq_h, xs_h, rt_h, W["q"], W["s"], W["bias"], cnt_h, bp_h,
                                    mpad)
    assert_within(g[live], g_ref[live], g_S[live], "raw mx8")
    if act == SWIGLU:
        h = bf16_host(gemm8(xq, xs, row_tok, Wd, counts, basep, tile_m, mpad, SWIGLU,
                            out=sentinel_out(mpad, N, SWIGLU)))
        assert_bf16_within_ulp(h[live], oracle.bf16_round(oracle.swiglu_oai(g[live], ALPHA, LIMIT)),
                               "swiglu mx8")
        assert np.all(h[~live] == SENT_BF16)


def test_deterministic_mx8():
    c = case(**MEDIUM)
    mpad, (counts, basep, row_tok, _), (cnt_h, bp_h, _, _) = front(c["ids"], c["E"], c["tile_m"])
    GU = moe.MX4Experts.from_numpy(c["gu"])
    xq, xs = moe.mx8_quantize(bf16_dev(c["x"]))
    outs = [host(gemm8(xq, xs, row_tok, GU, counts, basep, c["tile_m"], mpad, NONE))
            for _ in range(2)]
    live = live_mask(cnt_h, bp_h, mpad)
    assert np.array_equal(outs[0][live], outs[1][live])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill_pp512", "prefill_120b_t2048"])
def test_full_size_layer_mx8(name):
    # the layer at full size in the bench's launch configuration, every output: x and h
    # quantization bit-exact on all (live) rows; gate_up, h, down and y against the oracle
    wl = synth.WORKLOADS[name]
    log(f"full size mx8 {name}: E={wl.E} dim={wl.dim} ffn={wl.ffn} T={wl.T} k={wl.k}")
    tok = synth.tokens(wl, 0)
    W = synth.layer_weights(wl, 0)
    GU = moe.MX4Experts.from_numpy(W["gate_up"])
    DN = moe.MX4Experts.from_numpy(W["down"])
    out = moe.moe_layer(bf16_dev(tok["x"]), dev(tok["logits"]), GU, DN, wl.k, wl.tile_m, ALPHA,
                        LIMIT, projection="gemm_mx8")
    cnt_h, bp_h, rt_h, pos_h = (host(out[k]) for k in ("counts", "basep", "row_tok", "pos"))
    mpad = out["mpad"]
    live = live_mask(cnt_h, bp_h, mpad)
    F = wl.ffn
    xq_h, xs_h = host(out["xq"]), host(out["xs"])[:, :wl.dim // 32]
    assert_quant_equal(xq_h, host(out["xs"]), tok["x"], "x rows")

    # gate_up raw, every live output
    g = host(moe.mx4_moe_gemm_mx8(out["xq"], out["xs"], out["row_tok"], GU, out["counts"],
                                  out["basep"], wl.tile_m, mpad, NONE, ALPHA, LIMIT))
    log("  oracle gate_up")
    g_ref, S_g = oracle.project_mx8(xq_h, xs_h, rt_h, W["gate_up"]["q"], W["gate_up"]["s"],
                                    W["gate_up"]["bias"], cnt_h, bp_h, mpad)
    assert_within(g[live], g_ref[live], S_g[live], f"{name} gate_up mx8")
    # SwiGLU (the bf16 epilogue of the same call) from the GPU's own g and from the oracle's g
    h_bits = bf16_host(moe.mx4_moe_gemm_mx8(out["xq"], out["xs"], out["row_tok"], GU,
                                            out["counts"], out["basep"], wl.tile_m, mpad, SWIGLU,
                                            ALPHA, LIMIT))
    assert_bf16_within_ulp(h_bits[live],
                           oracle.bf16_round(oracle.swiglu_oai(g[live], ALPHA, LIMIT)),
                           f"{name} swiglu mx8 (GPU g)")
    assert_swiglu_within(h_bits[live], g_ref[live], S_g[live], F,
                         f"{name} swiglu mx8 (oracle g)", ALPHA, LIMIT)
    del g, g_ref, S_g
    # h as MXFP8 rows from the chain's epilogue: bit for bit the quantization of the bf16 rows
    hq_h, hs_h = host(out["hq"]), host(out["hs"])
    assert_quant_equal(hq_h[live], hs_h[live], h_bits[live], f"{name} h rows")
    # down from the GPU's hq, every live output
    d_h = host(out["d"])
    log("  oracle down")
    d_ref, d_S = oracle.project_mx8(hq_h, hs_h[:, :F // 32], None, W["down"]["q"],
                                    W["down"]["s"], W["down"]["bias"], cnt_h, bp_h, mpad)
    assert_within(d_h[live], d_ref[live], d_S[live], f"{name} down mx8")
    del d_ref, d_S
    # combine from the GPU's d, every token
    y_ref, y_S = oracle.combine(d_h, pos_h, host(out["w"]))
    assert_within(host(out["y"]), y_ref, y_S, f"{name} combine mx8")
