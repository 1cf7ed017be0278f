"""Parity of moe_router (router projection + top-k + bucket in one launch) with the oracle,
through the C ABI.

Protocol: the fp32 logits within |gpu - ref| <= 1e-3 * S + 1e-5 of oracle.router_logits; the
routing decisions taken on the GPU's own fp32 logits (ids, weights) and the CSR built from the
GPU's ids equal the oracle's route_topk and bucket bit for bit; the sync word is left zero.
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


def check_router(x, w, b, k, tile_m, want_logits=True, sync=None):
    import torch
    T, D = x.shape
    E = w.shape[0]
    if sync is None:
        sync = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = moe.moe_router(bf16_dev(x), bf16_dev(w), None if b is None else dev(b), k, tile_m, sync,
                         want_logits=True)
    torch.cuda.synchronize()
    assert int(host(sync)[0]) == 0, "sync word not left zero"
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
    "pp512": dict(T=512, D=2880, E=32, k=4, tile_m=16),
    "ragged": dict(T=37, D=96, E=8, k=2, tile_m=7),
    "wide_E128": dict(T=100, D=256, E=128, k=4, tile_m=16),
    "t2048_E128": dict(T=2048, D=2880, E=128, k=4, tile_m=16),
    "one_expert": dict(T=20, D=32, E=1, k=1, tile_m=4),
    "E_not_tile": dict(T=19, D=64, E=21, k=3, tile_m=5),
    "max_routed": dict(T=4096, D=64, E=64, k=4, tile_m=8),
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


def test_router_sync_word_reused_across_calls():
    import torch
    sync = torch.zeros(1, dtype=torch.int32, device="cuda")
    x, w, b = router_case(7, 100, 64, 32)
    for _ in range(3):
        check_router(x, w, b, 4, 16, sync=sync)
    x2, w2, b2 = router_case(8, 3, 64, 32)     # a smaller call on the same word
    check_router(x2, w2, b2, 2, 4, sync=sync)
