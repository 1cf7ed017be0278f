"""Parity of the HIP path (through the C ABI) with the CPU oracle, stage by stage.

Protocol: routing and the CSR are compared bit for bit; each expert projection is compared with
the oracle fed the same inputs the GPU stage received (the GPU's own previous-stage output), per
element within |gpu - ref| <= 1e-3 * S + 1e-5, S = |bias| + sum |a_i * w_i|; the SwiGLU output
within one bf16 ulp of the oracle's activation of the GPU's own fp32 gate_up result; exact-
arithmetic cases and the one-hot MXFP4 decode sweep must match exactly.
"""
import numpy as np
import pytest

import oracle
from mxfp4_mixture_experts_route_amd import _lib as moe
from mxfp4_mixture_experts_route_amd import synth
from helpers import (assert_bf16_within_ulp, assert_equal_values, assert_within, bf16_dev,
                     bf16_host, dev, host, live_mask)

pytestmark = pytest.mark.gpu

ALPHA, LIMIT = synth.ALPHA, synth.LIMIT
NONE, SWIGLU = moe.MOE_ACT_NONE, moe.MOE_ACT_SWIGLU_OAI
KERNELS = ["gemm", "gemv"]
SENT_F32 = 12345.0
SENT_BF16 = 0x4640   # 12288.0


def log(*a):
    print(*a, flush=True)


def proj(kernel, a, a_row, W, counts, basep, tile_m, mpad, act, out=None):
    fn = moe.mx4_moe_gemm if kernel == "gemm" else moe.mx4_moe_gemv
    return fn(a, a_row, W, counts, basep, tile_m, mpad, act, ALPHA, LIMIT, out=out)


def sentinel_out(mpad, N, act):
    import torch
    if act == SWIGLU:
        return torch.full((mpad, N // 2), SENT_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    return torch.full((mpad, N), SENT_F32, dtype=torch.float32, device="cuda")


def front(ids_np, E, tile_m):
    """moe_bucket on the GPU from given ids; returns device CSR + host copies."""
    k = ids_np.shape[1]
    T = ids_np.shape[0]
    mpad = moe.moe_mpad_max(T, k, E, tile_m)
    counts, basep, row_tok, pos = moe.moe_bucket(dev(ids_np.astype(np.int32)), E, tile_m, mpad)
    return mpad, (counts, basep, row_tok, pos), tuple(host(t) for t in (counts, basep, row_tok, pos))


def case(seed, E, D, F, T, k, tile_m, ids=None, bias=True):
    x = synth.random_bf16(seed, (T, D))
    logits = synth.random_logits(seed, T, E)
    gu = synth.random_mx4(seed * 7 + 1, E, 2 * F, D, bias_std=0.02 if bias else None)
    dn = synth.random_mx4(seed * 7 + 2, E, D, F, bias_std=0.02 if bias else None)
    if ids is None:
        ids, _ = oracle.route_topk(logits, k)
    return dict(x=x, logits=logits, gu=gu, dn=dn, ids=np.asarray(ids, np.int32), E=E, D=D, F=F,
                T=T, k=k, tile_m=tile_m)


MEDIUM = dict(seed=11, E=8, D=320, F=224, T=100, k=4, tile_m=16)


# ---------------------------------------------------------------------------------------------
# weight repack: a byte permutation, bit-exact against the layout's definition
# ---------------------------------------------------------------------------------------------

def chunked_reference(q, s):
    """The chunked layout written out with numpy: nibbles per expert chunk by chunk (blocks
    4c .. 4c+w_c-1 of all N rows, row after row); scales per expert in groups of 16 blocks, all
    N rows of a group together (16 bytes each), the last group zero-padded."""
    E, N, half_k = q.shape
    KB = half_k // 16
    qb = q.reshape(E, N, KB, 16)
    qo = []
    for e in range(E):
        for c0 in range(0, KB, 4):
            w = min(4, KB - c0)
            qo.append(qb[e, :, c0:c0 + w, :].reshape(-1))
    SP = (KB + 15) // 16 * 16
    rows = np.zeros((E, N, SP), dtype=np.uint8)
    rows[:, :, :KB] = s
    so = rows.reshape(E, N, SP // 16, 16).transpose(0, 2, 1, 3)   # [E][group][N][16]
    return np.concatenate(qo), np.ascontiguousarray(so).reshape(-1)


@pytest.mark.parametrize("E,N,K", [(3, 37, 160), (2, 16, 32), (4, 64, 2880), (1, 5, 96)])
def test_pack_matches_layout_definition(E, N, K):
    W = synth.random_mx4(E * N + K, E, N, K)
    log(f"pack E={E} N={N} K={K}")
    qp, sp = moe.mx4_pack_experts(dev(W["q"]), dev(W["s"]))
    q_ref, s_ref = chunked_reference(W["q"], W["s"])
    assert np.array_equal(host(qp).reshape(-1), q_ref)
    assert np.array_equal(host(sp).reshape(-1), s_ref)


# ---------------------------------------------------------------------------------------------
# routing and bucketing: bit-exact
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_route_and_bucket_bit_exact(name):
    wl = synth.WORKLOADS[name]
    tok = synth.tokens(wl)
    log(f"route/bucket {name}: T={wl.T} E={wl.E} k={wl.k} tile_m={wl.tile_m}")
    ids, w = moe.moe_route_topk(dev(tok["logits"]), wl.k)
    ids_ref, w_ref = oracle.route_topk(tok["logits"], wl.k)
    assert np.array_equal(host(ids), ids_ref)
    assert np.array_equal(host(w).view(np.uint32), w_ref.view(np.uint32))
    mpad, _, got = front(ids_ref, wl.E, wl.tile_m)
    ref = oracle.bucket(ids_ref, wl.E, wl.tile_m, mpad)
    for nm, g, r in zip(("counts", "basep", "row_tok", "pos"), got, ref):
        assert np.array_equal(g, r), nm
    if wl.n_dead:
        assert np.all(got[0][tok["dead"]] == 0)


@pytest.mark.parametrize("T,k,E,tile_m,skew", [(1, 4, 32, 1, 0.0), (1, 4, 32, 16, 0.0),
                                               (300, 1, 4, 16, 0.0), (777, 8, 64, 7, 2.0),
                                               (64, 4, 32, 32, 4.0), (5, 5, 5, 256, 0.0),
                                               (1000, 4, 1024, 16, 0.0),
                                               # T*k past the ids the kernel keeps in LDS, and
                                               # exactly at that limit
                                               (4000, 4, 64, 16, 1.0), (3072, 4, 128, 16, 0.0)])
def test_bucket_edge_shapes_bit_exact(T, k, E, tile_m, skew):
    ids = synth.random_ids(T + E, T, k, E, skew=skew)
    log(f"bucket T={T} k={k} E={E} tile_m={tile_m}")
    mpad, _, got = front(ids, E, tile_m)
    ref = oracle.bucket(ids, E, tile_m, mpad)
    for nm, g, r in zip(("counts", "basep", "row_tok", "pos"), got, ref):
        assert np.array_equal(g, r), nm


def test_stale_runtime_error_is_not_a_launch_failure():
    """An error state left in the HIP runtime by an earlier, unrelated call (a host-side
    hipSetDevice with an invalid ordinal) is not reported as the next call's launch failure."""
    import ctypes
    hip_path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line)
    hip = ctypes.CDLL(hip_path)
    assert hip.hipSetDevice(ctypes.c_int(1 << 20)) != 0
    ids = synth.random_ids(5, 4, 2, 8)
    mpad, _, got = front(ids, 8, 16)   # raised MoeError(MOE_ELAUNCH) on the stale error
    for nm, g, r in zip(("counts", "basep", "row_tok", "pos"), got, oracle.bucket(ids, 8, 16, mpad)):
        assert np.array_equal(g, r), nm


def test_route_ties_and_signed_zero():
    logits = np.array([[1.0, 3.0, 3.0, -1.0], [-1.0, 0.0, -0.0, -2.0], [0.25] * 4,
                       [-0.0, 0.0, -0.0, 0.0]], dtype=np.float32)
    for k in (1, 2, 4):
        ids, w = moe.moe_route_topk(dev(logits), k)
        ids_ref, w_ref = oracle.route_topk(logits, k)
        assert np.array_equal(host(ids), ids_ref)
        assert np.array_equal(host(w), w_ref)


@pytest.mark.parametrize("kernel", KERNELS)
def test_swiglu_epilogue_over_the_gate_range(kernel):
    """Zero activations make g the bias row exactly, so the fused epilogue's h is SwiGLU-OAI of
    chosen (gate, up) pairs: gates from -200 to 10 (h down to bf16's smallest subnormals and
    below, where the hardware exp2 underflows), ups across both clamps; within one bf16 ulp."""
    F = 4096
    g = np.random.default_rng(5)
    gate = np.concatenate([np.linspace(-200.0, 10.0, F - 64), g.uniform(-95, -80, 64)])
    up = g.uniform(-9.0, 9.0, F)
    bias = np.concatenate([gate, up]).astype(np.float32)[None, :]
    W = {"q": g.integers(0, 256, (1, 2 * F, 16)).astype(np.uint8),
         "s": np.full((1, 2 * F, 1), 127, np.uint8), "bias": bias}
    x = np.zeros((3, 32), dtype=np.uint16)
    ids = np.zeros((3, 1), dtype=np.int32)
    log(f"swiglu range {kernel}")
    mpad, (counts, basep, row_tok, _), (cnt_h, bp_h, _, _) = front(ids, 1, 16)
    live = live_mask(cnt_h, bp_h, mpad)
    h = bf16_host(proj(kernel, bf16_dev(x), row_tok, moe.MX4Experts.from_numpy(W), counts, basep,
                       16, mpad, SWIGLU))
    ref = oracle.bf16_round(oracle.swiglu_oai(bias.astype(np.float64), ALPHA, LIMIT))
    assert_bf16_within_ulp(h[live], np.repeat(ref, int(live.sum()), axis=0), f"{kernel} h")


@pytest.mark.parametrize("E,k", [(32, 4), (64, 8), (100, 4), (1024, 16)])
def test_route_nan_rows_give_experts_in_range(E, k):
    """NaN logits rank below every number (a total order): rows with NaNs, all-NaN rows and
    -inf route to k distinct ids in [0, E), bit for bit the oracle's; both rank paths (E <= 64
    and the arg-best rounds past 64)."""
    g = np.random.default_rng(E + k)
    logits = (np.round(g.standard_normal((24, E)) * 2) / 2).astype(np.float32)
    logits[g.random((24, E)) < 0.4] = np.nan
    logits[g.random((24, E)) < 0.05] = -np.inf
    logits[0] = np.nan
    logits[1, :] = -np.inf
    logits[2, : E // 2] = np.nan
    log(f"route NaN rows E={E} k={k}")
    ids, w = moe.moe_route_topk(dev(logits), k)
    ids_ref, w_ref = oracle.route_topk(logits, k)
    got = host(ids)
    assert got.min() >= 0 and got.max() < E
    assert np.array_equal(got, ids_ref)
    wg = host(w)
    assert np.array_equal(np.isnan(wg), np.isnan(w_ref))
    assert np.array_equal(np.nan_to_num(wg), np.nan_to_num(w_ref))


# ---------------------------------------------------------------------------------------------
# staged projections on a case that spans several tiles with ragged tails
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", KERNELS)
def test_staged_chain_medium(kernel):
    c = case(**MEDIUM)
    E, D, F, tile_m = c["E"], c["D"], c["F"], c["tile_m"]
    log(f"staged chain {kernel}: E={E} D={D} F={F} T={c['T']} k={c['k']}")
    mpad, (counts, basep, row_tok, pos), (cnt_h, bp_h, rt_h, pos_h) = front(c["ids"], E, tile_m)
    live = live_mask(cnt_h, bp_h, mpad)
    GU = moe.MX4Experts.from_numpy(c["gu"])
    DN = moe.MX4Experts.from_numpy(c["dn"])
    x = bf16_dev(c["x"])

    # gate_up raw (act NONE): g within tolerance; rows that are not live stay untouched
    g = proj(kernel, x, row_tok, GU, counts, basep, tile_m, mpad, NONE,
             out=sentinel_out(mpad, 2 * F, NONE))
    g_h = host(g)
    g_ref, g_S = oracle.project(c["x"], rt_h, c["gu"]["q"], c["gu"]["s"], c["gu"]["bias"],
                                cnt_h, bp_h, mpad)
    assert_within(g_h[live], g_ref[live], g_S[live], "gate_up")
    assert np.all(g_h[~live] == SENT_F32)

    # SwiGLU epilogue: h within 1 bf16 ulp of the oracle's activation of the GPU's own g
    h = proj(kernel, x, row_tok, GU, counts, basep, tile_m, mpad, SWIGLU,
             out=sentinel_out(mpad, 2 * F, SWIGLU))
    h_bits = bf16_host(h)
    h_ref = oracle.bf16_round(oracle.swiglu_oai(g_h[live].astype(np.float64), ALPHA, LIMIT))
    assert_bf16_within_ulp(h_bits[live], h_ref, "swiglu")
    assert np.all(h_bits[~live] == SENT_BF16)

    # down from the GPU's bf16 h (rows already in CSR order)
    d = proj(kernel, h, None, DN, counts, basep, tile_m, mpad, NONE,
             out=sentinel_out(mpad, D, NONE))
    d_h = host(d)
    d_ref, d_S = oracle.project(h_bits, None, c["dn"]["q"], c["dn"]["s"], c["dn"]["bias"],
                                cnt_h, bp_h, mpad)
    assert_within(d_h[live], d_ref[live], d_S[live], "down")
    assert np.all(d_h[~live] == SENT_F32)

    # combine from the GPU's d
    wts = oracle.route_topk(c["logits"], c["k"])[1]
    y = moe.moe_combine(d, pos, dev(wts))
    y_ref, y_S = oracle.combine(d_h, pos_h, wts)
    assert_within(host(y), y_ref, y_S, "combine")

    # end to end from inputs only (h may differ by a bf16 rounding flip; loose, informational)
    full = oracle.chain(c["x"], c["logits"], c["gu"], c["dn"], c["k"], tile_m, ALPHA, LIMIT)
    assert_within(host(y), full["y"], full["y_S"], "chain end-to-end", rel=2e-2)


@pytest.mark.parametrize("kernel", KERNELS)
def test_deterministic(kernel):
    c = case(**MEDIUM)
    mpad, (counts, basep, row_tok, pos), _ = front(c["ids"], c["E"], c["tile_m"])
    GU = moe.MX4Experts.from_numpy(c["gu"])
    x = bf16_dev(c["x"])
    outs = [bf16_host(proj(kernel, x, row_tok, GU, counts, basep, c["tile_m"], mpad, SWIGLU))
            for _ in range(2)]
    live = live_mask(*(host(t) for t in (counts, basep)), mpad)
    assert np.array_equal(outs[0][live], outs[1][live])


# ---------------------------------------------------------------------------------------------
# exact arithmetic: every partial sum is exact, so GPU == oracle exactly
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", KERNELS)
def test_exact_arithmetic(kernel):
    g = np.random.default_rng(3)
    E, D, F, T, k, tile_m = 5, 160, 96, 40, 3, 16
    x = synth.round_f32_to_bf16_bits(g.integers(-4, 5, (T, D)).astype(np.float32))
    gu = {"q": g.integers(0, 256, (E, 2 * F, D // 2)).astype(np.uint8),
          "s": g.integers(126, 128, (E, 2 * F, D // 32)).astype(np.uint8),
          "bias": (g.integers(-8, 9, (E, 2 * F)) / 4).astype(np.float32)}
    dn = {"q": g.integers(0, 256, (E, D, F // 2)).astype(np.uint8),
          "s": g.integers(126, 128, (E, D, F // 32)).astype(np.uint8),
          "bias": (g.integers(-8, 9, (E, D)) / 4).astype(np.float32)}
    ids = synth.random_ids(9, T, k, E)
    log(f"exact arithmetic {kernel}")
    mpad, (counts, basep, row_tok, _), (cnt_h, bp_h, rt_h, _) = front(ids, E, tile_m)
    live = live_mask(cnt_h, bp_h, mpad)
    out = host(proj(kernel, bf16_dev(x), row_tok, moe.MX4Experts.from_numpy(gu), counts, basep,
                    tile_m, mpad, NONE))
    ref, _ = oracle.project(x, rt_h, gu["q"], gu["s"], gu["bias"], cnt_h, bp_h, mpad)
    assert_equal_values(out[live], ref[live], "gate_up exact")
    # down on an integer-valued h in CSR order
    hx = np.zeros((mpad, F), dtype=np.uint16)
    hx[live] = synth.round_f32_to_bf16_bits(g.integers(-4, 5, (int(live.sum()), F)).astype(np.float32))
    out = host(proj(kernel, bf16_dev(hx), None, moe.MX4Experts.from_numpy(dn), counts, basep,
                    tile_m, mpad, NONE))
    ref, _ = oracle.project(hx, None, dn["q"], dn["s"], dn["bias"], cnt_h, bp_h, mpad)
    assert_equal_values(out[live], ref[live], "down exact")


# ---------------------------------------------------------------------------------------------
# the MXFP4 decode through the real kernels: all 16 codes x 256 scale bytes, one-hot activations
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", KERNELS)
def test_one_hot_decode_sweep(kernel):
    K = 32
    N = 2 * 16 * 256
    q = np.zeros((1, N, K // 2), dtype=np.uint8)
    s = np.zeros((1, N, 1), dtype=np.uint8)
    for half in range(2):
        for c in range(16):
            for e in range(256):
                n = half * 4096 + c * 256 + e
                if half == 0:
                    q[0, n, 0] = c              # element 0 (low nibble of byte 0)
                else:
                    q[0, n, 15] = c << 4        # element 31 (high nibble of byte 15)
                s[0, n, 0] = e
    x = np.zeros((2, K), dtype=np.float32)
    x[0, 0] = 1.0
    x[1, 31] = 1.0
    xb = synth.round_f32_to_bf16_bits(x)
    ids = np.zeros((2, 1), dtype=np.int32)
    log(f"one-hot sweep {kernel}")
    mpad, (counts, basep, row_tok, _), (cnt_h, bp_h, rt_h, _) = front(ids, 1, 1)
    W = {"q": q, "s": s, "bias": None}
    out = host(proj(kernel, bf16_dev(xb), row_tok, moe.MX4Experts.from_numpy(W), counts, basep,
                    1, mpad, NONE))
    with np.errstate(invalid="ignore", over="ignore"):
        ref, _ = oracle.project(xb, rt_h, q, s, None, cnt_h, bp_h, mpad)
    assert_equal_values(out[:2], ref[:2], "one-hot decode")


# ---------------------------------------------------------------------------------------------
# shape edge cases
# ---------------------------------------------------------------------------------------------

def skewed_ids(counts_per_expert, seed):
    ids = np.concatenate([np.full(c, e, dtype=np.int32) for e, c in enumerate(counts_per_expert)])
    np.random.default_rng(seed).shuffle(ids)
    return ids[:, None]


EDGE = {
    "single_block_K32": dict(seed=1, E=4, D=32, F=32, T=9, k=2, tile_m=16),
    "one_token": dict(seed=2, E=32, D=64, F=64, T=1, k=4, tile_m=1),
    "empty_expert": dict(seed=3, E=8, D=64, F=64, T=20, k=2, tile_m=16,
                         ids=synth.random_ids(3, 20, 2, 7)),          # expert 7 gets nothing
    "all_on_one_expert": dict(seed=4, E=4, D=64, F=64, T=300, k=1, tile_m=16,
                              ids=np.full((300, 1), 2, dtype=np.int32)),
    "counts_around_granules": dict(seed=5, E=6, D=64, F=64, T=456, k=1, tile_m=16,
                                   ids=skewed_ids([15, 16, 17, 135, 136, 137], 5)),
    "tile_m_7": dict(seed=6, E=5, D=96, F=64, T=33, k=3, tile_m=7),
    # tall passes: 256 rows = two full 128-row passes; 320 = two plus a 64-row remainder pass;
    # 136 rows on one expert beside a 32-row one (a full pass plus an 8-row remainder)
    "m256_one_expert": dict(seed=8, E=3, D=64, F=64, T=256, k=1, tile_m=16,
                            ids=np.full((256, 1), 1, dtype=np.int32)),
    "m320_one_expert": dict(seed=9, E=3, D=96, F=64, T=320, k=1, tile_m=16,
                            ids=np.full((320, 1), 2, dtype=np.int32)),
    "m136_and_32": dict(seed=10, E=4, D=64, F=96, T=168, k=1, tile_m=16,
                        ids=skewed_ids([0, 136, 0, 32], 10)),
    "tile_m_32": dict(seed=7, E=16, D=64, F=96, T=70, k=4, tile_m=32),
    # the GEMM deals experts to XCDs by cost for E <= 64 and in id order above: both sides of
    # the boundary, with every expert live and with fewer live experts than placement slots
    "E64_cost_order": dict(seed=12, E=64, D=64, F=64, T=200, k=4, tile_m=16),
    "E65_id_order": dict(seed=13, E=65, D=64, F=64, T=200, k=4, tile_m=16),
    "E64_few_live": dict(seed=14, E=64, D=64, F=96, T=40, k=1, tile_m=16,
                         ids=skewed_ids([0] * 50 + [7, 5, 0, 9, 3, 0, 11, 5] + [0] * 6, 14)),
}


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases(kernel, name):
    c = case(**EDGE[name])
    E, D, F, tile_m = c["E"], c["D"], c["F"], c["tile_m"]
    log(f"edge {name} {kernel}: E={E} D={D} F={F} T={c['T']} k={c['k']} tile_m={tile_m}")
    mpad, (counts, basep, row_tok, pos), (cnt_h, bp_h, rt_h, _) = front(c["ids"], E, tile_m)
    live = live_mask(cnt_h, bp_h, mpad)
    GU = moe.MX4Experts.from_numpy(c["gu"])
    DN = moe.MX4Experts.from_numpy(c["dn"])
    x = bf16_dev(c["x"])
    g = host(proj(kernel, x, row_tok, GU, counts, basep, tile_m, mpad, NONE,
                  out=sentinel_out(mpad, 2 * F, NONE)))
    g_ref, g_S = oracle.project(c["x"], rt_h, c["gu"]["q"], c["gu"]["s"], c["gu"]["bias"],
                                cnt_h, bp_h, mpad)
    assert_within(g[live], g_ref[live], g_S[live], "gate_up")
    assert np.all(g[~live] == SENT_F32)
    h = proj(kernel, x, row_tok, GU, counts, basep, tile_m, mpad, SWIGLU,
             out=sentinel_out(mpad, 2 * F, SWIGLU))
    h_bits = bf16_host(h)
    assert_bf16_within_ulp(h_bits[live], oracle.bf16_round(oracle.swiglu_oai(g[live], ALPHA, LIMIT)),
                           "swiglu")
    assert np.all(h_bits[~live] == SENT_BF16)
    d = host(proj(kernel, h, None, DN, counts, basep, tile_m, mpad, NONE,
                  out=sentinel_out(mpad, D, NONE)))
    d_ref, d_S = oracle.project(h_bits, None, c["dn"]["q"], c["dn"]["s"], c["dn"]["bias"],
                                cnt_h, bp_h, mpad)
    assert_within(d[live], d_ref[live], d_S[live], "down")
    assert np.all(d[~live] == SENT_F32)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("N,K,act", [(40, 64, NONE), (36, 64, SWIGLU), (264, 96, NONE),
                                     (2 * 130, 64, SWIGLU), (8, 32, NONE), (2, 32, SWIGLU)])
def test_projection_ragged_n(kernel, N, K, act):
    # N not a multiple of the 16-row tile (or of 4 for the vector stores)
    E, T, k, tile_m = 3, 25, 2, 16
    W = synth.random_mx4(N + K, E, N, K)
    xb = synth.random_bf16(N, (T, K))
    ids = synth.random_ids(N, T, k, E)
    log(f"ragged {kernel} N={N} K={K} act={act}")
    mpad, (counts, basep, row_tok, _), (cnt_h, bp_h, rt_h, _) = front(ids, E, tile_m)
    live = live_mask(cnt_h, bp_h, mpad)
    Wd = moe.MX4Experts.from_numpy(W)
    g = host(proj(kernel, bf16_dev(xb), row_tok, Wd, counts, basep, tile_m, mpad, NONE))
    g_ref, g_S = oracle.project(xb, rt_h, W["q"], W["s"], W["bias"], cnt_h, bp_h, mpad)
    assert_within(g[live], g_ref[live], g_S[live], "raw")
    if act == SWIGLU:
        h = bf16_host(proj(kernel, bf16_dev(xb), row_tok, Wd, counts, basep, tile_m, mpad, SWIGLU,
                           out=sentinel_out(mpad, N, SWIGLU)))
        assert_bf16_within_ulp(h[live], oracle.bf16_round(oracle.swiglu_oai(g[live], ALPHA, LIMIT)),
                               "swiglu")
        assert np.all(h[~live] == SENT_BF16)


def test_gemv_and_gemm_agree_on_the_same_call():
    c = case(**MEDIUM)
    mpad, (counts, basep, row_tok, _), (cnt_h, bp_h, _, _) = front(c["ids"], c["E"], c["tile_m"])
    live = live_mask(cnt_h, bp_h, mpad)
    GU = moe.MX4Experts.from_numpy(c["gu"])
    x = bf16_dev(c["x"])
    a = host(proj("gemm", x, row_tok, GU, counts, basep, c["tile_m"], mpad, NONE))
    b = host(proj("gemv", x, row_tok, GU, counts, basep, c["tile_m"], mpad, NONE))
    _, S = oracle.project(c["x"], host(row_tok), c["gu"]["q"], c["gu"]["s"], c["gu"]["bias"],
                          cnt_h, bp_h, mpad)
    assert_within(a[live], b[live], S[live], "gemm vs gemv", rel=2e-3)
