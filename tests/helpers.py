"""Shared helpers of the GPU parity tests: device transfer, the tolerance checks, and running the
routing/bucketing front of the chain through the C ABI."""
from __future__ import annotations

import numpy as np

import oracle

REL_TOL = 1e-3     # |gpu - ref| <= REL_TOL * S + ABS_TOL, S = |bias| + sum |a_i * w_i|
ABS_TOL = 1e-5


def torch_mod():
    import torch
    return torch


def dev(a):
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if not a.flags.writeable:   # torch wants a writable array even to copy it
        a = a.copy()
    return torch.from_numpy(a).to("cuda")


def bf16_dev(bits):
    torch = torch_mod()
    return dev(np.asarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def host(t):
    return t.detach().cpu().numpy()


def bf16_host(t):
    torch = torch_mod()
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_within(gpu, ref, S, what: str, rel: float = REL_TOL, abs_: float = ABS_TOL):
    """Element-wise |gpu - ref| <= rel*S + abs_ (the chain's fp32-accumulation tolerance).
    NaN must meet NaN, and infinities must match exactly."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    nan_ok = np.isnan(gpu) & np.isnan(ref)
    inf_ref = np.isinf(ref)
    with np.errstate(invalid="ignore"):
        ok = nan_ok | (inf_ref & (gpu == ref)) | (~inf_ref & (np.abs(gpu - ref) <= rel * S + abs_))
    if not np.all(ok):
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} outside tolerance; first at {i}: "
                             f"gpu={gpu[i]!r} ref={ref[i]!r} S={S[i]!r}")


def assert_equal_values(gpu, ref, what: str):
    """Numerically equal (NaN meets NaN; -0 == +0): the exact-arithmetic cases."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ok = (gpu == ref) | (np.isnan(gpu) & np.isnan(ref))
    if not np.all(ok):
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} differ; first at {i}: "
                             f"gpu={gpu[i]!r} ref={ref[i]!r}")


def bf16_ulp(bits) -> np.ndarray:
    """Spacing of bf16 values at each bf16 bit pattern (2^-133 in the subnormal range)."""
    v = np.abs(oracle.bf16_to_f64(bits))
    _, e = np.frexp(np.where(v > 0, v, 1.0))
    return np.where(v >= 2.0 ** -126, np.ldexp(1.0, e - 8), 2.0 ** -133)


def assert_bf16_within_ulp(gpu_bits, ref_bits, what: str, ulps: int = 1):
    g = oracle.bf16_to_f64(gpu_bits)
    r = oracle.bf16_to_f64(ref_bits)
    ok = (np.isnan(g) & np.isnan(r)) | (np.abs(g - r) <= ulps * bf16_ulp(ref_bits))
    if not np.all(ok):
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} beyond {ulps} bf16 ulp; first at "
                             f"{i}: gpu={g[i]!r} ref={r[i]!r}")


def live_mask(counts, basep, mpad):
    m = np.zeros(mpad, dtype=bool)
    for e in range(len(counts)):
        m[basep[e]:basep[e] + counts[e]] = True
    return m


def assert_swiglu_within(h_bits, g_ref, S_g, F, what, alpha, limit):
    """bf16 h from a fused gate_up epilogue (no fp32 intermediate to stage from) against the
    SwiGLU-OAI of the oracle's own gate_up rows g_ref [rows][2F]: within one bf16 ulp of the
    exact activation plus the gate_up tolerance carried through it (|dh/dgate| <= 1.1*(|uc|+1)
    <= 8.8 and |dh/dup| <= limit where the input is not clamped)."""
    g_ref = np.asarray(g_ref, dtype=np.float64)
    S_g = np.asarray(S_g, dtype=np.float64)
    tol_g = REL_TOL * S_g[:, :F] + ABS_TOL
    tol_u = REL_TOL * S_g[:, F:] + ABS_TOL
    ref = oracle.swiglu_oai(g_ref, alpha, limit)
    got = oracle.bf16_to_f64(h_bits)
    bound = bf16_ulp(oracle.bf16_round(ref)) + 8.8 * tol_g + limit * tol_u
    ok = np.abs(got - ref) <= bound
    if not np.all(ok):
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside; first at {i}: "
                             f"got={got[i]} ref={ref[i]} bound={bound[i]}")
