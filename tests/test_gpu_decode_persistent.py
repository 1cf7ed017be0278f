"""Parity of the one-launch decode layer (mx4_moe_decode_persistent) with the CPU oracle, by the
protocol of the two-launch tests: routing and CSR bit for bit; h within one bf16 ulp plus the
gate_up tolerance carried through SwiGLU-OAI; d from the GPU's own h and y from the GPU's own d
within |gpu - ref| <= 1e-3 * S + 1e-5. Also: the workspace counters are re-zeroed with no error flag, a
capped grid (workgroups taking several items in turn) gives the same routing and in-tolerance
outputs, and d and y equal the two-launch path's bit for bit whenever h does.
"""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_mixture_experts_route_amd import _lib as moe
from mxfp4_mixture_experts_route_amd import synth
from helpers import assert_within, bf16_dev, bf16_host, dev, host
from test_gpu_decode import CASES, check_h, make_case

pytestmark = pytest.mark.gpu

ALPHA, LIMIT = synth.ALPHA, synth.LIMIT


def log(*a):
    print(*a, flush=True)


def new_ws():
    return torch.zeros(moe.MOE_DECODE_WS_WORDS, dtype=torch.int32, device="cuda")


def run_persistent(c, ws=None, max_wg=0):
    GU = moe.MX4Experts.from_numpy(c["gu"])
    DN = moe.MX4Experts.from_numpy(c["dn"])
    ws = new_ws() if ws is None else ws
    out = moe.mx4_moe_decode_persistent(dev(c["logits"]), bf16_dev(c["x"]), GU, DN, c["k"], ws,
                                        ALPHA, LIMIT, want_d=True, max_workgroups=max_wg)
    torch.cuda.synchronize()
    wsh = host(ws)
    assert wsh[3] == 0, "a wait ran past its bound"
    # the completion counters are zero again after every call (only the epoch words advance)
    assert wsh[0] == 0 and not wsh[32:288:32].any(), f"counters not re-zeroed: {wsh[:8]}"
    return out


def check_against_oracle(c, out, what):
    E, F, T, k = c["E"], c["F"], c["T"], c["k"]
    ids_ref, w_ref = oracle.route_topk(c["logits"], k)
    assert np.array_equal(host(out["ids"]), ids_ref), what
    assert np.array_equal(host(out["w"]).view(np.uint32), w_ref.view(np.uint32)), what
    mpad = T * k
    cnt, bp, rt, pos = oracle.bucket(ids_ref, E, 1, mpad)
    for nm, ref in (("counts", cnt), ("basep", bp), ("row_tok", rt), ("pos", pos)):
        assert np.array_equal(host(out[nm]), ref), f"{what} {nm}"
    pos_flat = pos.reshape(-1)
    h_bits = bf16_host(out["h"])
    g_ref, S_g = oracle.project(c["x"], rt, c["gu"]["q"], c["gu"]["s"], c["gu"]["bias"], cnt, bp,
                                mpad)
    check_h(h_bits, g_ref, S_g, pos_flat, F, f"{what} h")
    h_csr = np.zeros_like(h_bits)
    h_csr[pos_flat] = h_bits
    d_ref, S_d = oracle.project(h_csr, None, c["dn"]["q"], c["dn"]["s"], c["dn"]["bias"], cnt, bp,
                                mpad)
    d_h = host(out["d"])
    assert_within(d_h, d_ref[pos_flat], S_d[pos_flat], f"{what} d")
    y_ref, y_S = oracle.combine(d_h, np.arange(T * k, dtype=np.int32).reshape(T, k), w_ref)
    assert_within(host(out["y"]), y_ref, y_S, f"{what} y")


@pytest.mark.parametrize("name", list(CASES))
def test_persistent_parity(name):
    c = make_case(**CASES[name])
    log(f"persistent decode {name}: E={c['E']} D={c['D']} F={c['F']} T={c['T']} k={c['k']}")
    out = run_persistent(c)
    check_against_oracle(c, out, name)
    # with the same h, d and y are those of the two-launch path bit for bit
    two = moe.mx4_moe_decode(dev(c["logits"]), bf16_dev(c["x"]), moe.MX4Experts.from_numpy(c["gu"]),
                             moe.MX4Experts.from_numpy(c["dn"]), c["k"], ALPHA, LIMIT, want_d=True)
    if np.array_equal(bf16_host(out["h"]), bf16_host(two["h"])):
        assert np.array_equal(host(out["d"]).view(np.uint32), host(two["d"]).view(np.uint32))
        assert np.array_equal(host(out["y"]).view(np.uint32), host(two["y"]).view(np.uint32))


@pytest.mark.parametrize("max_wg", [1, 3, 7])
def test_persistent_capped_grid(max_wg):
    # a few workgroups take every item in turn: gate_up items first, then down items that wait
    c = make_case(**CASES["medium_T5"])
    log(f"persistent decode, grid capped at {max_wg}")
    check_against_oracle(c, run_persistent(c, max_wg=max_wg), f"cap {max_wg}")


def test_persistent_workspace_reused_and_deterministic():
    ws = new_ws()
    c = make_case(**CASES["max_T16"])
    a = run_persistent(c, ws=ws)
    b = run_persistent(c, ws=ws)
    small = make_case(**CASES["one_token_E32_k4"])
    check_against_oracle(small, run_persistent(small, ws=ws), "after reuse")
    c2 = run_persistent(c, ws=ws)
    assert np.array_equal(bf16_host(a["h"]), bf16_host(b["h"]))
    assert np.array_equal(bf16_host(a["h"]), bf16_host(c2["h"]))
    for key in ("d", "y"):
        assert np.array_equal(host(a[key]).view(np.uint32), host(b[key]).view(np.uint32)), key
        assert np.array_equal(host(a[key]).view(np.uint32), host(c2[key]).view(np.uint32)), key


@pytest.mark.timeout(600)
def test_persistent_full_size_gptoss_t1():
    """The bench's decode layer (gpt-oss-20b shape, T = 1): routing exact; every h value
    against the activation of the oracle's gate_up rows, every d value against the oracle from
    the GPU's h, y against the oracle combine of the GPU's d."""
    wl = synth.WORKLOADS["decode_t1"]
    tok = synth.tokens(wl, 0)
    W = synth.layer_weights(wl, 0)
    log(f"persistent decode full size: E={wl.E} dim={wl.dim} ffn={wl.ffn} k={wl.k}")
    c = dict(x=tok["x"], logits=tok["logits"], gu=W["gate_up"], dn=W["down"], E=wl.E, D=wl.dim,
             F=wl.ffn, T=1, k=wl.k)
    out = run_persistent(c)
    ids_ref, w_ref = oracle.route_topk(tok["logits"], wl.k)
    assert np.array_equal(host(out["ids"]), ids_ref)
    cnt, bp, rt, pos = oracle.bucket(ids_ref, wl.E, 1, wl.k)
    pos_flat = pos.reshape(-1)
    h_bits = bf16_host(out["h"])
    g_ref, S_g = oracle.project(tok["x"], rt, W["gate_up"]["q"], W["gate_up"]["s"],
                                W["gate_up"]["bias"], cnt, bp, wl.k)
    check_h(h_bits, g_ref, S_g, pos_flat, wl.ffn, "full-size persistent h")
    h_csr = np.zeros_like(h_bits)
    h_csr[pos_flat] = h_bits
    d_ref, d_S = oracle.project(h_csr, None, W["down"]["q"], W["down"]["s"], W["down"]["bias"],
                                cnt, bp, wl.k)
    d_h = host(out["d"])
    assert_within(d_h, d_ref[pos_flat], d_S[pos_flat], "full-size persistent d")
    y_ref, y_S = oracle.combine(d_h, np.arange(wl.k, dtype=np.int32).reshape(1, wl.k), w_ref)
    assert_within(host(out["y"]), y_ref, y_S, "full-size persistent y")
