"""mx4_moe_decode_persistent_static (the library's own workspace, nothing allocated) against
mx4_moe_decode_persistent (the caller's workspace) on the same inputs.

Two static calls in a row, the second with a smaller input (the library's array keeps the first
call's contents). Each call's outputs equal the workspace entry point's bit for bit (same kernel,
same grid) and meet the oracle bar: routing and CSR bit-exact, h within one bf16 ulp plus the
carried gate_up tolerance, d and y within |gpu - ref| <= 1e-3 * S + 1e-5.
"""
import numpy as np
import pytest
import torch

from mxfp4_mixture_experts_route_amd import _lib as moe
from helpers import bf16_dev, dev, host
from test_gpu_decode import CASES, make_case
from test_gpu_decode_persistent import check_against_oracle, new_ws

pytestmark = pytest.mark.gpu

ALPHA, LIMIT = 1.702, 7.0
KEYS = ("ids", "w", "counts", "basep", "row_tok", "pos", "h", "d", "y")


def log(*a):
    print(*a, flush=True)


def outputs(c):
    """Output tensors of one call, filled with a sentinel so that an unwritten value shows."""
    T, E, k, F, D = c["T"], c["E"], c["k"], c["F"], c["D"]
    spec = {"ids": ((T, k), torch.int32), "w": ((T, k), torch.float32),
            "counts": ((E,), torch.int32), "basep": ((E + 1,), torch.int32),
            "row_tok": ((T * k,), torch.int32), "pos": ((T, k), torch.int32),
            "h": ((T * k, F), torch.int16), "d": ((T * k, D), torch.float32),
            "y": ((T, D), torch.float32)}
    o = {}
    for key, (shape, dt) in spec.items():
        o[key] = torch.full(shape, 77, dtype=dt, device="cuda")
    o["h"] = o["h"].view(torch.bfloat16)
    return o


def as_bits(t):
    a = host(t.view(torch.int16) if t.dtype == torch.bfloat16 else t)
    return a.view(np.uint16) if a.dtype == np.int16 else a.view(np.uint32)


def test_static_workspace_matches_caller_workspace_two_calls():
    cases = [make_case(**CASES["max_T16"]), make_case(**CASES["one_token_E32_k4"])]
    prepared = []
    for c in cases:
        prepared.append(dict(c=c, logits=dev(c["logits"]), x=bf16_dev(c["x"]),
                             GU=moe.MX4Experts.from_numpy(c["gu"]),
                             DN=moe.MX4Experts.from_numpy(c["dn"])))
    # the two static calls back to back, the second smaller
    static_out = []
    for p in prepared:
        c = p["c"]
        log(f"static-workspace decode: E={c['E']} D={c['D']} F={c['F']} T={c['T']} k={c['k']}")
        o = outputs(c)
        moe.mx4_moe_decode_persistent_static(p["logits"], p["x"], p["GU"], p["DN"], c["k"], o,
                                             ALPHA, LIMIT)
        static_out.append(o)
    torch.cuda.synchronize()
    for p, o in zip(prepared, static_out):
        c = p["c"]
        ref = outputs(c)
        moe.mx4_moe_decode_persistent(p["logits"], p["x"], p["GU"], p["DN"], c["k"], new_ws(),
                                      ALPHA, LIMIT, want_d=True, out=ref)
        torch.cuda.synchronize()
        for key in KEYS:
            assert np.array_equal(as_bits(o[key]), as_bits(ref[key])), f"T={c['T']} {key}"
        check_against_oracle(c, o, f"static T={c['T']}")
