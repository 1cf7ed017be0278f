"""Parity of the fused decode chain (mx4_moe_decode, two launches) with the CPU oracle.

Routing and the CSR (tile_m = 1) must match bit for bit. h has no fp32 intermediate to stage
from, so it is checked against the oracle's activation of the oracle's gate_up result, within
one bf16 ulp plus the gate_up tolerance carried through SwiGLU-OAI (|dh/dgate| <= 1.1*(|uc|+1)
<= 8.8 and |dh/dup| <= limit = 7 where not clamped). d is checked against the oracle fed the
GPU's own h, y against the oracle combine of the GPU's own d, both within
|gpu - ref| <= 1e-3 * S + 1e-5. The fused kernels run the same per-row arithmetic as the CSR
calls, so h, d and y must also equal the five-call chain (gemv, tile_m = 1) bit for bit.
"""
import numpy as np
import pytest

import oracle
from mxfp4_mixture_experts_route_amd import _lib as moe
from mxfp4_mixture_experts_route_amd import synth
from helpers import REL_TOL, ABS_TOL, assert_within, bf16_dev, bf16_host, bf16_ulp, dev, host

pytestmark = pytest.mark.gpu

ALPHA, LIMIT = synth.ALPHA, synth.LIMIT


def log(*a):
    print(*a, flush=True)


def make_case(seed, E, D, F, T, k, logit_std=1.0):
    return dict(x=synth.random_bf16(seed, (T, D)),
                logits=(synth.random_logits(seed, T, E) * np.float32(logit_std)).astype(np.float32),
                gu=synth.random_mx4(seed * 7 + 1, E, 2 * F, D, bias_std=0.02),
                dn=synth.random_mx4(seed * 7 + 2, E, D, F, bias_std=0.02), E=E, D=D, F=F, T=T, k=k)


CASES = {
    "tiny_T8_k2": dict(seed=0, E=4, D=64, F=64, T=8, k=2),
    "one_token_E32_k4": dict(seed=21, E=32, D=64, F=64, T=1, k=4),
    "medium_T5": dict(seed=22, E=8, D=320, F=224, T=5, k=4),
    "max_T16": dict(seed=23, E=8, D=128, F=96, T=16, k=4),
    "max_k8": dict(seed=24, E=16, D=64, F=64, T=3, k=8),
    "single_expert": dict(seed=25, E=1, D=32, F=32, T=2, k=1),
    "ksplit_both": dict(seed=26, E=6, D=1600, F=416, T=2, k=3),     # D: 13 chunks (split)
    "long_ffn": dict(seed=27, E=4, D=96, F=1664, T=1, k=2),         # F: 13 chunks (split)
    # routing inside the gate_up launch: logits row by LDS-DMA for E <= 64, loaded per lane above
    "E64_k4": dict(seed=29, E=64, D=64, F=64, T=3, k=4),
    "E128_k4": dict(seed=30, E=128, D=64, F=64, T=2, k=4),
}


def check_h(h_bits, g_ref, S_g, pos_flat, F, what):
    """h (routed-row order) against SwiGLU-OAI of the oracle's gate_up rows."""
    g = g_ref[pos_flat]
    S = S_g[pos_flat]
    gate, up = g[:, :F], g[:, F:]
    tol_g = REL_TOL * S[:, :F] + ABS_TOL
    tol_u = REL_TOL * S[:, F:] + ABS_TOL
    ref = oracle.swiglu_oai(g, ALPHA, LIMIT)   # fp64
    got = oracle.bf16_to_f64(h_bits)
    bound = bf16_ulp(oracle.bf16_round(ref)) + 8.8 * tol_g + LIMIT * tol_u
    ok = np.abs(got - ref) <= bound
    if not np.all(ok):
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} outside; first at {i}: got={got[i]} "
                             f"ref={ref[i]} bound={bound[i]} gate={gate[i]} up={up[i]}")


def run_and_check(c, against_csr=True):
    E, D, F, T, k = c["E"], c["D"], c["F"], c["T"], c["k"]
    GU = moe.MX4Experts.from_numpy(c["gu"])
    DN = moe.MX4Experts.from_numpy(c["dn"])
    logits_d, x_d = dev(c["logits"]), bf16_dev(c["x"])
    out = moe.mx4_moe_decode(logits_d, x_d, GU, DN, k, ALPHA, LIMIT, want_d=True)

    ids_ref, w_ref = oracle.route_topk(c["logits"], k)
    assert np.array_equal(host(out["ids"]), ids_ref)
    w_got = host(out["w"])   # bit for bit; a NaN weight (NaN logits) meets a NaN of any payload
    assert np.array_equal(np.isnan(w_got), np.isnan(w_ref))
    assert np.array_equal(np.where(np.isnan(w_got), 0, w_got).view(np.uint32),
                          np.where(np.isnan(w_ref), 0, w_ref).astype(np.float32).view(np.uint32))
    mpad = T * k
    cnt, bp, rt, pos = oracle.bucket(ids_ref, E, 1, mpad)
    for nm, ref in (("counts", cnt), ("basep", bp), ("row_tok", rt), ("pos", pos)):
        assert np.array_equal(host(out[nm]), ref), nm
    pos_flat = pos.reshape(-1)

    h_bits = bf16_host(out["h"])
    g_ref, S_g = oracle.project(c["x"], rt, c["gu"]["q"], c["gu"]["s"], c["gu"]["bias"], cnt, bp,
                                mpad)
    check_h(h_bits, g_ref, S_g, pos_flat, F, "fused h")

    # d from the GPU's own h: put the routed rows into CSR order for the oracle
    h_csr = np.zeros_like(h_bits)
    h_csr[pos_flat] = h_bits
    d_ref_csr, S_d_csr = oracle.project(h_csr, None, c["dn"]["q"], c["dn"]["s"], c["dn"]["bias"],
                                        cnt, bp, mpad)
    d_h = host(out["d"])
    assert_within(d_h, d_ref_csr[pos_flat], S_d_csr[pos_flat], "fused d")

    # y from the GPU's own d (routed-row order: pos = identity)
    y_ref, y_S = oracle.combine(d_h, np.arange(T * k, dtype=np.int32).reshape(T, k), w_ref)
    y = host(out["y"])
    assert_within(y, y_ref, y_S, "fused y")

    if against_csr:
        ref = moe.moe_layer(x_d, logits_d, GU, DN, k, 1, ALPHA, LIMIT, projection="gemv")
        assert np.array_equal(h_bits, bf16_host(ref["h"])[pos_flat]), "h vs CSR chain"
        assert np.array_equal(d_h.view(np.uint32), host(ref["d"])[pos_flat].view(np.uint32)), \
            "d vs CSR chain"
        assert np.array_equal(y.view(np.uint32), host(ref["y"]).view(np.uint32)), "y vs CSR chain"
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_decode_fused_parity(name):
    c = make_case(**CASES[name])
    log(f"fused decode {name}: E={c['E']} D={c['D']} F={c['F']} T={c['T']} k={c['k']}")
    run_and_check(c)


def test_decode_without_d_and_deterministic():
    c = make_case(**CASES["medium_T5"])
    GU = moe.MX4Experts.from_numpy(c["gu"])
    DN = moe.MX4Experts.from_numpy(c["dn"])
    logits_d, x_d = dev(c["logits"]), bf16_dev(c["x"])
    a = moe.mx4_moe_decode(logits_d, x_d, GU, DN, c["k"], ALPHA, LIMIT)
    b = moe.mx4_moe_decode(logits_d, x_d, GU, DN, c["k"], ALPHA, LIMIT, want_d=True)
    assert "d" not in a
    assert np.array_equal(host(a["y"]).view(np.uint32), host(b["y"]).view(np.uint32))
    assert np.array_equal(bf16_host(a["h"]), bf16_host(b["h"]))


def test_decode_ties_route_like_route_topk():
    c = make_case(seed=28, E=8, D=64, F=64, T=4, k=3)
    c["logits"][0] = 0.5                      # all tied: ids 0, 1, 2
    c["logits"][1, [2, 5]] = 9.0              # tie at the top
    c["logits"][2] = -0.0
    c["logits"][2, 3] = 0.0
    run_and_check(c)


@pytest.mark.parametrize("E", [32, 128])
def test_decode_nan_logits_route_in_range(E):
    """A token whose logits row is NaN (all or part) routes to k distinct experts in [0, E), the
    oracle's order; the fused kernels then stream those experts' rows (finite x, so h, d and y
    are finite and within tolerance)."""
    c = make_case(31 + E, E=E, D=64, F=64, T=4, k=4)
    c["logits"][0] = np.nan
    c["logits"][1, ::3] = np.nan
    c["logits"][2] = -np.inf
    log(f"decode NaN logits E={E}")
    out = run_and_check(c, against_csr=False)
    ids = host(out["ids"])
    assert ids.min() >= 0 and ids.max() < E


@pytest.mark.timeout(600)
def test_decode_full_size_gptoss_t1():
    """The bench's decode layer (gpt-oss-20b shape, T = 1) against the oracle on every output,
    and whole against the five-call chain."""
    wl = synth.WORKLOADS["decode_t1"]
    tok = synth.tokens(wl, 0)
    W = synth.layer_weights(wl, 0)
    log(f"fused decode full size: E={wl.E} dim={wl.dim} ffn={wl.ffn} k={wl.k}")
    GU = moe.MX4Experts.from_numpy(W["gate_up"])
    DN = moe.MX4Experts.from_numpy(W["down"])
    logits_d, x_d = dev(tok["logits"]), bf16_dev(tok["x"])
    out = moe.mx4_moe_decode(logits_d, x_d, GU, DN, wl.k, ALPHA, LIMIT, want_d=True)
    ids_ref, w_ref = oracle.route_topk(tok["logits"], wl.k)
    assert np.array_equal(host(out["ids"]), ids_ref)
    assert np.array_equal(host(out["w"]).view(np.uint32), w_ref.view(np.uint32))
    cnt, bp, rt, pos = oracle.bucket(ids_ref, wl.E, 1, wl.k)
    for nm, ref in (("counts", cnt), ("basep", bp), ("row_tok", rt), ("pos", pos)):
        assert np.array_equal(host(out[nm]), ref), nm
    pos_flat = pos.reshape(-1)
    h_bits = bf16_host(out["h"])
    # every h value against the activation of the oracle's gate_up rows
    g_ref, S_g = oracle.project(tok["x"], rt, W["gate_up"]["q"], W["gate_up"]["s"],
                                W["gate_up"]["bias"], cnt, bp, wl.k)
    check_h(h_bits, g_ref, S_g, pos_flat, wl.ffn, "full-size fused h")
    # every d value from the GPU's h
    h_csr = np.zeros_like(h_bits)
    h_csr[pos_flat] = h_bits
    d_ref, d_S = oracle.project(h_csr, None, W["down"]["q"], W["down"]["s"], W["down"]["bias"],
                                cnt, bp, wl.k)
    d_h = host(out["d"])
    assert_within(d_h, d_ref[pos_flat], d_S[pos_flat], "full-size fused d")
    y_ref, y_S = oracle.combine(d_h, np.arange(wl.k, dtype=np.int32).reshape(1, wl.k), w_ref)
    assert_within(host(out["y"]), y_ref, y_S, "full-size fused y")
    ref = moe.moe_layer(x_d, logits_d, GU, DN, wl.k, 1, ALPHA, LIMIT, projection="gemv")
    assert np.array_equal(host(out["y"]).view(np.uint32), host(ref["y"]).view(np.uint32))
