"""Parity of moe_router (router projection + top-k + bucket in one launch) with the oracle,
through the C ABI.

Protocol: the fp32 logits within |gpu - ref| <= 1e-3 * S + 1e-5 of oracle.router_logits; the
routing decisions taken on the GPU's own fp32 logits (ids, weights) and the CSR built from the
GPU's ids equal the oracle's route_topk and bucket bit for bit; the workspace's counter word is
left zero. A few tokens (T <= 16, E <= 256) take the split-reduction kernel, more the
one-workgroup-per-16-tokens kernel (for E >= 64 a pair of workgroups per 16 tokens, each with
half of the experts, whose top-k candidates the later one merges), whose last workgroup builds
the CSR from per-group histograms (or, when their table does not fit its LDS, by sweeping all ids
per expert); each is covered, and one workspace serves both kernels in turn. Every counter word
of the workspace is left zero.
"""
import numpy as np
import pytest

import oracle
from mxfp4_mixture_experts_route_amd import _lib as moe
from mxfp4_mixture_experts_route_amd import synth
from helpers import assert_within, bf16_dev, dev, host

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)


def router_case(seed, T, D, E, bias=True, dup_rows=()):
    g = np.random.default_rng(seed)
    x = synth.round_f32_to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    w = g.standard_normal((E, D)).astype(np.float32) / np.float32(np.sqrt(D))
    for a, b in dup_rows:                     # equal router rows: exactly tied logits
        w[b] = w[a]
    w = synth.round_f32_to_bf16_bits(w)
    b = (g.standard_normal(E) * 0.1).astype(np.float32) if bias else None
    if b is not None:
        for a, c in dup_rows:
            b[c] = b[a]
    return x, w, b


def new_ws():
    import torch
    return torch.zeros(moe.MOE_ROUTER_WS_WORDS, dtype=torch.int32, device="cuda")


def check_router(x, w, b, k, tile_m, want_logits=True, ws=None):
    import torch
    T, D = x.shape
    E = w.shape[0]
    if ws is None:
        ws = new_ws()
    out = moe.moe_router(bf16_dev(x), bf16_dev(w), None if b is None else dev(b), k, tile_m, ws,
                         want_logits=True)
    torch.cuda.synchronize()
    wsh = host(ws)
    assert int(wsh[0]) == 0, "counter word not left zero"
    assert int(abs(wsh[64:1088]).max()) == 0, "pair counters not left zero"
    lg = host(out["logits"])
    ref, S = oracle.router_logits(x, w, b)
    assert_within(lg, ref, S, "router logits")
    ids_ref, w_ref = oracle.route_topk(lg, k)
    assert np.array_equal(host(out["ids"]), ids_ref), "ids"
    assert np.array_equal(host(out["w"]), w_ref), "weights"
    mpad = out["mpad"]
    for name, r in zip(("counts", "basep", "row_tok", "pos"),
                       oracle.bucket(ids_ref, E, tile_m, mpad)):
        assert np.array_equal(host(out[name]), r), name
    return out


CASES = {
    "decode_T1": dict(T=1, D=2880, E=32, k=4, tile_m=1),
    # split reduction: every token in one tile, E up to 256, ragged E and D
    "split_T16_E256": dict(T=16, D=2880, E=256, k=8, tile_m=16),
    "split_T3_E21": dict(T=3, D=96, E=21, k=3, tile_m=4),
    "split_T7_E128_D64": dict(T=7, D=64, E=128, k=4, tile_m=1),
    "split_T1_E1": dict(T=1, D=32, E=1, k=1, tile_m=1),
    # just past the split kernel's limits: the one-workgroup-per-tile kernel
    "T17_E32": dict(T=17, D=2880, E=32, k=4, tile_m=1),
    "T2_E257": dict(T=2, D=64, E=257, k=4, tile_m=1),
    "pp512": dict(T=512, D=2880, E=32, k=4, tile_m=16),
    "ragged": dict(T=37, D=96, E=8, k=2, tile_m=7),
    "wide_E128": dict(T=100, D=256, E=128, k=4, tile_m=16),
    "t2048_E128": dict(T=2048, D=2880, E=128, k=4, tile_m=16),
    "one_expert": dict(T=20, D=32, E=1, k=1, tile_m=4),
    "E_not_tile": dict(T=19, D=64, E=21, k=3, tile_m=5),
    "max_routed": dict(T=4096, D=64, E=64, k=4, tile_m=8),
    # in-group ranks over 16 picks per token, T*k at the limit
    "k16_max_routed": dict(T=1024, D=32, E=64, k=16, tile_m=4),
    # odd E on the grouped path: the last table word holds one expert
    "grouped_E255": dict(T=40, D=64, E=255, k=5, tile_m=3),
    # per-group table past its LDS budget: every expert sweeps all ids
    "sweep_E1024": dict(T=600, D=32, E=1024, k=4, tile_m=3),
}


@pytest.mark.parametrize("name", list(CASES))
def test_router_bit_exact_routing(name):
    c = CASES[name]
    log(f"router {name}: {c}")
    x, w, b = router_case(11 + list(CASES).index(name), c["T"], c["D"], c["E"])
    check_router(x, w, b, c["k"], c["tile_m"])


def test_router_without_bias_and_ties():
    # duplicated router rows tie exactly; the lower expert id wins
    x, w, b = router_case(5, 40, 128, 16, bias=False, dup_rows=((3, 9), (4, 5), (0, 15)))
    out = check_router(x, w, b, 4, 16)
    lg = host(out["logits"])
    assert np.array_equal(lg[:, 3], lg[:, 9]) and np.array_equal(lg[:, 4], lg[:, 5])


def test_router_workspace_reused_across_calls():
    ws = new_ws()
    x, w, b = router_case(7, 100, 64, 32)
    for _ in range(3):
        check_router(x, w, b, 4, 16, ws=ws)
    x2, w2, b2 = router_case(8, 3, 64, 32)     # a smaller call (split kernel) on the same words
    a = check_router(x2, w2, b2, 2, 4, ws=ws)
    b_ = check_router(x2, w2, b2, 2, 4, ws=ws)   # deterministic: the same partial-sum order
    assert np.array_equal(host(a["logits"]).view(np.uint32), host(b_["logits"]).view(np.uint32))
    check_router(x, w, b, 4, 16, ws=ws)        # and back to the multi-workgroup kernel
