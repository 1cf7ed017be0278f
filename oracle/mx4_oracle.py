"""CPU oracle of the routed MXFP4 expert chain (gpt-oss routed experts).

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import or run this module. It shares no code with the HIP library (no kernels, headers, tables
or helpers) and never imports it; both sides only share the seeded input generator, which holds
none of the chain's arithmetic.

Everything here is the plain definition of each step, written for a reader to check by eye:
per-token / per-row loops, float64 arithmetic, and numpy's matmul as the only library primitive.
The chain stores some values in narrower types, and the oracle reproduces exactly those
roundings: routing weights are f32, decoded MXFP4 weights are fp32 values, and the SwiGLU
output h is bf16 (round-to-nearest-even) before the down projection.

Sources (web pages on the daScript repository's dasLLAMA engine):
  [fusion] PR #3579 "dasLLAMA gpt-oss arc", commit log, the Metal fusion-lane commit (bucket pass
           with the padded-prefix base computed per expert; expert matmul seeded from the bias
           row; SwiGLU-OAI that skips ghost rows past the last padded bucket end).
  [chain]  PR #3579, commit log, the fused MoE expert chain commit, and the PR body's section
           "Fused MoE expert chain" (gate and up rows + bias + activation; down rows + bias;
           routing-weighted sum in slot order).
  [mx4]    PR #3558 "dasLLAMA: dig the last two board reds green", section "gpt-oss: mx4 kernels
           to the lab-winning shape" and its ladder table (16-value e2m1 table; e8m0 exponent
           byte decoded bit-exactly for all 256 values, subnormal results included).
  [lattice] PR #3579, commit log, the lattice shift commit: MXFP4 nibbles are unpacked with a
           15 mask (low nibble) and a right shift by 4 (high nibble).
Facts the pages leave open are filled from outside sources, marked [ext]: the OCP Microscaling
(MX) v1.0 e2m1 / e8m0 definitions and the public gpt-oss model (softmax over the k selected
logits; the clamped SwiGLU with alpha = 1.702 and limit = 7).

Readings where the pages are silent (each pinned in tests/test_oracle_pins.py):
  - element 2i of a row is the low nibble of byte i, element 2i+1 the high nibble;
  - e8m0 byte 255 decodes to NaN; a decoded weight beyond the fp32 range is +-inf;
  - top-k ties go to the lower expert id, and a NaN logit ranks below every number (a total
    order); weights = softmax of the k selected logits in double, rounded to f32;
  - CSR rows within a bucket are in ascending token order; padding/ghost rows hold -1;
  - gate_up rows [0, F) are the gate, rows [F, 2F) the up projection;
  - the router is a linear layer with bias over bf16 rows ([ext, gpt-oss]), bf16 weights;
  - MXFP8 activations (the MX-scaled MFMA variant; [ext] OCP 8-bit FP and MX v1.0): an all-zero
    block takes the smallest scale; elements round to nearest even and saturate at 448; the
    projection is the MX dot product (each block's exact sum scaled, result stored as fp32), so
    a zero activation times a weight beyond the fp32 range contributes 0.

Every function is pinned (closed forms, invariants, brute force, exact arithmetic); none is
"parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------------------------
# MXFP4 decode
# --------------------------------------------------------------------------------------------

# [ext] OCP MX v1.0 FP4 E2M1: bit 3 = sign, bits 2..1 = exponent (bias 1), bit 0 = mantissa.
# [mx4] the kernels decode through a 16-value table indexed by the 4-bit code.
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                       -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)


def e2m1_decode(codes) -> np.ndarray:
    """Value of each 4-bit e2m1 code ([mx4] 16-value table; [ext] OCP MX v1.0)."""
    codes = np.asarray(codes)
    return E2M1_TABLE[codes if codes.dtype == np.uint8 else codes.astype(np.int64)]


def e8m0_decode(e) -> np.ndarray:
    """Scale of each e8m0 byte: 2^(e-127); byte 255 is NaN ([mx4]: every one of the 256 bytes
    decodes exactly, subnormal results included; [ext] OCP MX v1.0 for 255)."""
    e = np.asarray(e, dtype=np.int64)
    out = np.ldexp(np.ones(e.shape, dtype=np.float64), (e - 127).astype(np.int32))
    return np.where(e == 255, np.nan, out)


def unpack_codes(q: np.ndarray) -> np.ndarray:
    """e2m1 codes of packed rows [..., K/2] -> [..., K]: element 2i = low nibble of byte i,
    element 2i+1 = high nibble ([lattice]: low via a 15 mask, high via a shift by 4)."""
    q = np.asarray(q, dtype=np.uint8)
    lo = q & np.uint8(15)
    hi = q >> np.uint8(4)
    codes = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), dtype=np.uint8)
    codes[..., 0::2] = lo
    codes[..., 1::2] = hi
    return codes


def dequant_exact(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Decoded MXFP4 matrix [..., N, K] as exact float64 values: e2m1(code) * 2^(s-127) for the
    32-element block holding the element ([mx4]); NaN where the scale byte is 255. A float64
    holds every such product exactly (2 significant bits, exponents -128..130)."""
    codes = unpack_codes(q)
    K = codes.shape[-1]
    scale = np.repeat(e8m0_decode(s), 32, axis=-1)
    assert scale.shape[-1] == K
    return e2m1_decode(codes) * scale


def dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Decoded MXFP4 matrix [..., N, K] as fp32 values, the operand of the bf16-activation
    projections: dequant_exact's values stored as fp32, which overflows to +-inf beyond the fp32
    range (reading; in range the value is exact in fp32 and in bf16 alike)."""
    with np.errstate(over="ignore", invalid="ignore"):
        return dequant_exact(q, s).astype(np.float32)


# --------------------------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Round float64 values to bf16 (8 significant bits, fp32 exponent range), nearest-even,
    returned as bit patterns. Written from the format's definition: the spacing of bf16 values
    near |x| is 2^(e-8) with frexp exponent e, floored at the subnormal spacing 2^-133; values
    that round to 2^128 or beyond are infinite."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    finite = np.isfinite(a) & (a > 0)
    _, e = np.frexp(np.where(finite, a, 1.0))
    quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.where(finite, np.rint(a / quantum) * quantum, a)        # rint: half to even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    with np.errstate(over="ignore"):
        bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.signbit(x), bits | np.uint16(0x8000), bits)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)


# --------------------------------------------------------------------------------------------
# MXFP8 activations (the variant of the projections on the MX-scaled MFMA). The pages quantize
# only the weights; every fact of this section is [ext]: the OCP 8-bit floating point spec
# (E4M3) and the OCP MX v1.0 spec (its conversion of a 32-value block to a shared e8m0 scale
# plus elements).
# --------------------------------------------------------------------------------------------

E4M3_MAX = 448.0   # largest finite E4M3 magnitude: exponent field 15, mantissa 110


def e4m3_decode(codes) -> np.ndarray:
    """Value of each FP8 E4M3 byte [ext]: bit 7 = sign, bits 6..3 = exponent (bias 7), bits
    2..0 = mantissa; exponent field 0 holds the subnormals m * 2^-9; the two bytes with all of
    bits 6..0 set are NaN; there are no infinities."""
    c = np.asarray(codes, dtype=np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int32)))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


# magnitude -> code of the 127 finite non-negative E4M3 values
_E4M3_CODE_OF = {float(v): c for c, v in enumerate(e4m3_decode(np.arange(127)))}


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code of each finite float64 value, ties to the even mantissa, magnitudes
    beyond the largest finite value saturating to it (the MX conversion clamps instead of
    producing NaN) [ext]. Written from the format: values near |v| are spaced 2^(e-4) apart
    for frexp exponent e, floored at the subnormal spacing 2^-9. The sign bit is the value's,
    so -0.0 and negatives that round to zero give 0x80."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    quantum = np.ldexp(1.0, np.maximum(e, -5) - 4)
    r = np.minimum(np.rint(a / quantum) * quantum, E4M3_MAX)       # rint: half to even
    mag = np.array([_E4M3_CODE_OF[float(x)] for x in r.ravel()], dtype=np.int64).reshape(r.shape)
    return (mag | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def mx8_quantize(a_bits):
    """MXFP8 (E4M3 elements) of bf16 rows [rows][K] -> (codes u8 [rows][K], scales u8
    [rows][K/32]) by the OCP MX v1.0 conversion [ext]: for each block of 32 consecutive values,
    the shared exponent is floor(log2(max |v|)) minus 8 (the exponent of E4M3's largest
    normal), clamped to e8m0's range [-127, 127]; each element is e4m3_encode(v / 2^X), exact
    division by a power of two. Reading (the spec leaves it free): an all-zero block takes the
    smallest scale, X = -127 (the clamp of log2(0) = -inf). Inputs must be finite."""
    a = bf16_to_f64(a_bits)
    rows, K = a.shape
    assert K % 32 == 0
    blocks = a.reshape(rows, K // 32, 32)
    amax = np.abs(blocks).max(axis=-1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))                  # amax in [2^(e-1), 2^e)
    X = np.where(amax > 0, np.clip(e - 1 - 8, -127, 127), -127)
    codes = e4m3_encode(blocks / np.ldexp(1.0, X.astype(np.int32))[..., None])
    return codes.reshape(rows, K), (X + 127).astype(np.uint8)


def mx8_dequant(codes, scales) -> np.ndarray:
    """Values of MXFP8 rows: e4m3(code) * 2^(s-127) for the element's 32-value block, float64
    (exact)."""
    return e4m3_decode(codes) * np.repeat(e8m0_decode(scales), 32, axis=-1)


# --------------------------------------------------------------------------------------------
# routing and bucketing
# --------------------------------------------------------------------------------------------

def router_logits(x_bits, w_bits, bias=None) -> np.ndarray:
    """Router projection: logits[t][e] = bias[e] + sum_d x[t][d] * W_r[e][d], x bf16 [T][D],
    W_r bf16 [E][D], bias f32 [E] or None; float64 (products of bf16 values are exact, only the
    sum rounds, at float64). [ext, gpt-oss] the router is a linear layer with bias; the pages
    start the chain from its output (the per-token expert ids). Also returns S = |bias| +
    sum_d |x[t][d] * W_r[e][d]|, the scale of the fp32 summation error bound."""
    x = bf16_to_f64(x_bits)
    W = bf16_to_f64(w_bits)
    b = np.zeros(W.shape[0]) if bias is None else np.asarray(bias, dtype=np.float64)
    return b[None, :] + x @ W.T, np.abs(b)[None, :] + np.abs(x) @ np.abs(W).T


def _beats(a: float, b: float) -> bool:
    """Logit a ranks strictly above logit b: a number above a NaN, else the larger number."""
    if math.isnan(a) or math.isnan(b):
        return math.isnan(b) and not math.isnan(a)
    return a > b


def _exp(v: float) -> float:
    """e^v, NaN for NaN (math.exp raises on nothing here: v <= 0 or NaN)."""
    return math.nan if math.isnan(v) else math.exp(v)


def route_topk(logits: np.ndarray, k: int):
    """Top-k routing of each token.

    ids: the k largest logits, descending; equal logits ordered by ascending expert id
    ([chain] names per-token expert ids; [mx4] k = 4 at gpt-oss shape; tie order is a reading).
    A NaN logit ranks below every number, -inf included, and NaNs among themselves by id
    (reading: the pages route finite logits; this makes the order total, so any row yields k
    distinct experts).
    w: softmax over the k selected logits [ext, gpt-oss router], w_s = exp(l_s - l_0) /
    sum_j exp(l_j - l_0) in float64, summed in slot order, rounded to f32 (NaN wherever a NaN
    logit enters the sum).
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    assert 1 <= k <= E
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    for t in range(T):
        remaining = list(range(E))
        chosen = []
        for _ in range(k):
            best = remaining[0]
            for e in remaining[1:]:
                if _beats(float(logits[t, e]), float(logits[t, best])):  # strict: ties keep lower id
                    best = e
            chosen.append(best)
            remaining.remove(best)
        ids[t] = chosen
        l0 = float(logits[t, chosen[0]])
        num = [_exp(float(logits[t, e]) - l0) for e in chosen]
        den = 0.0
        for v in num:
            den += v
        w[t] = [np.float32(v / den) for v in num]
    return ids, w


def mpad_max(T: int, k: int, E: int, tile_m: int) -> int:
    """CSR row capacity: R = T*k rows plus at most tile_m-1 padding rows for each of at most
    min(E, R) non-empty experts, rounded up to tile_m ([fusion]: mpad, the padded row count)."""
    R = T * k
    n = R + min(E, R) * (tile_m - 1)
    return -(-n // tile_m) * tile_m


def bucket(ids: np.ndarray, E: int, tile_m: int, mpad: int):
    """Bucket/CSR of routed rows per expert with padded prefix bases ([fusion]).

    counts[e] = #(t,s) with ids[t][s] = e; basep[0] = 0, basep[e+1] = basep[e] +
    roundup(counts[e], tile_m); expert e's rows are its (t,s) in ascending t (reading: the
    order of a serial scan), row_tok[basep[e]+j] = t_j, pos[t][s] = that row; padding rows and
    ghost rows [basep[E], mpad) hold -1.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        assert len(set(ids[t].tolist())) == k, "a token picks an expert at most once"
        for s in range(k):
            counts[ids[t, s]] += 1
    basep = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        basep[e + 1] = basep[e] + -(-counts[e] // tile_m) * tile_m
    assert basep[E] <= mpad
    row_tok = np.full(mpad, -1, dtype=np.int64)
    pos = np.empty((T, k), dtype=np.int64)
    fill = basep[:E].copy()
    for t in range(T):
        for s in range(k):
            e = ids[t, s]
            row_tok[fill[e]] = t
            pos[t, s] = fill[e]
            fill[e] += 1
    return (counts.astype(np.int32), basep.astype(np.int32), row_tok.astype(np.int32),
            pos.astype(np.int32))


# --------------------------------------------------------------------------------------------
# expert projections
# --------------------------------------------------------------------------------------------

def live_rows(counts, basep):
    """(expert, CSR row) of every live row: rows [basep[e], basep[e] + counts[e])."""
    out = []
    for e in range(len(counts)):
        for j in range(int(counts[e])):
            out.append((e, int(basep[e]) + j))
    return out


def project(a_bits, a_row, q, s, bias, counts, basep, mpad: int):
    """Bias-seeded MXFP4 projection of every live CSR row ([fusion]: accumulator starts at the
    expert's bias row; [chain]: rows + bias).

    out[r][n] = bias[e][n] + sum_i x_r[i] * W[e][n][i] with x_r = a[a_row[r]] (or a[r] when
    a_row is None), in float64 (products of bf16 and decoded fp32 values are exact; only the
    sum rounds, at float64). Also returns S[r][n] = |bias| + sum_i |x_r[i] * W[e][n][i]|, the
    scale of the fp32 summation error bound. Rows that are not live are NaN in both.
    """
    return project_values(bf16_to_f64(a_bits), a_row, q, s, bias, counts, basep, mpad)


# Smallest magnitude that an fp32 store rounds (to nearest even) to infinity: halfway between
# the largest finite fp32 value (2 - 2^-23) * 2^127 and 2^128.
FP32_OVERFLOW = (2.0 - 2.0 ** -24) * 2.0 ** 127


def round_fp32_range(v: np.ndarray) -> np.ndarray:
    """float64 values as an fp32 result holds them in range: magnitudes at or beyond
    FP32_OVERFLOW become +-inf; everything else is left at float64 precision (the tolerance
    covers the fp32 rounding)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        return np.where(np.abs(v) >= FP32_OVERFLOW, np.copysign(np.inf, v), v)


def project_mx8(a_codes, a_scales, a_row, q, s, bias, counts, basep, mpad: int):
    """The projection of `project` with MXFP8 activation rows (codes [rows][K], scales
    [rows][K/32], as mx8_quantize returns them) in place of bf16 rows: x_r is the exact value of
    the quantized row.

    The product follows the OCP MX v1.0 dot product [ext]: each pair of 32-value blocks
    contributes its exact sum of element products times the two blocks' scales, and the result
    is stored as fp32. So the weights are taken at their exact values (dequant_exact: a decoded
    weight beyond the fp32 range is a finite number here, and a zero activation times it is
    0), every product x_i * w_i is exact in float64, the sum rounds at float64, and the result
    is rounded into the fp32 range (round_fp32_range). A block with scale byte 255 is NaN, and
    so is every output it enters. Partial sums that would overflow fp32 on the way are not
    modelled (no test input reaches the fp32 range except through a single block)."""
    out, S = project_values(mx8_dequant(a_codes, a_scales), a_row, q, s, bias, counts, basep,
                            mpad, weights=dequant_exact)
    return round_fp32_range(out), S


def project_values(a, a_row, q, s, bias, counts, basep, mpad: int, weights=None):
    """The projection of `project` with the activation rows given as float64 values [rows][K]
    and the weights decoded by `weights` (default: dequant, fp32 values)."""
    weights = dequant if weights is None else weights
    E, N, _ = q.shape
    K = q.shape[2] * 2
    out = np.full((mpad, N), np.nan, dtype=np.float64)
    S = np.full((mpad, N), np.nan, dtype=np.float64)
    for e in range(E):
        c = int(counts[e])
        if c == 0:
            continue
        rows = int(basep[e]) + np.arange(c)
        src = rows if a_row is None else np.asarray(a_row)[rows]
        x = a[src]                                                  # [c][K]
        W = weights(q[e], s[e]).astype(np.float64)                  # [N][K]
        b = np.zeros(N) if bias is None else np.asarray(bias[e], dtype=np.float64)
        with np.errstate(invalid="ignore", over="ignore"):
            out[rows] = b[None, :] + x @ W.T
            S[rows] = np.abs(b)[None, :] + np.abs(x) @ np.abs(W).T
        assert x.shape[1] == K
    return out, S


def project_at(a_bits, a_row, q, s, bias, counts, basep, samples):
    """The same projection as `project`, evaluated only at the sampled (row, n) pairs (rows must
    be live). For checks of single outputs where the whole product is not needed."""
    a = np.asarray(a_bits)
    return _project_at(lambda src: bf16_to_f64(a[src]), a_row, q, s, bias, counts, basep,
                       samples, dequant)


def project_mx8_at(a_codes, a_scales, a_row, q, s, bias, counts, basep, samples):
    """project_mx8 evaluated only at the sampled (row, n) pairs (rows must be live)."""
    vals, S = _project_at(lambda src: mx8_dequant(a_codes[src], a_scales[src]), a_row, q, s,
                          bias, counts, basep, samples, dequant_exact)
    return round_fp32_range(vals), S


def _project_at(row_values, a_row, q, s, bias, counts, basep, samples, weights):
    basep = np.asarray(basep)
    counts = np.asarray(counts)
    vals = np.empty(len(samples), dtype=np.float64)
    S = np.empty(len(samples), dtype=np.float64)
    for i, (r, n) in enumerate(samples):
        e = int(np.searchsorted(basep, r, side="right") - 1)
        assert basep[e] <= r < basep[e] + counts[e], "sampled row is not live"
        src = r if a_row is None else int(a_row[r])
        x = row_values(src)
        w = weights(q[e, n][None, :], s[e, n][None, :])[0].astype(np.float64)
        b = 0.0 if bias is None else float(bias[e, n])
        with np.errstate(invalid="ignore", over="ignore"):
            vals[i] = b + float(np.dot(x, w))
            S[i] = abs(b) + float(np.dot(np.abs(x), np.abs(w)))
    return vals, S


# --------------------------------------------------------------------------------------------
# SwiGLU-OAI and combine
# --------------------------------------------------------------------------------------------

def swiglu_oai(g, alpha: float, limit: float) -> np.ndarray:
    """Clamped SwiGLU-OAI of gate_up rows g [rows][2F] -> float64 [rows][F] ([fusion] names the
    swiglu_oai activation; [ext, gpt-oss] the form): gate = g[:, :F], up = g[:, F:],
    gc = min(gate, limit), uc = clamp(up, -limit, limit), out = gc * sigmoid(alpha*gc) * (uc+1),
    sigmoid(z) = 1 / (1 + e^-z)."""
    g = np.asarray(g, dtype=np.float64)
    F = g.shape[-1] // 2
    gate, up = g[..., :F], g[..., F:]
    gc = np.minimum(gate, limit)
    uc = np.clip(up, -limit, limit)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-alpha * gc))
    return gc * sig * (uc + 1.0)


def combine(d, pos, w):
    """Router-weighted combine in slot order ([chain]): y[t] = sum_s w[t][s] * d[pos[t][s]],
    float64. Also returns S = sum_s |w[t][s] * d[pos[t][s]]|."""
    d = np.asarray(d)    # only the rows pos names are read (the others may hold anything)
    pos = np.asarray(pos)
    w = np.asarray(w, dtype=np.float64)
    T, k = pos.shape
    y = np.zeros((T, d.shape[1]), dtype=np.float64)
    S = np.zeros((T, d.shape[1]), dtype=np.float64)
    for t in range(T):
        for s_ in range(k):
            term = w[t, s_] * np.asarray(d[pos[t, s_]], dtype=np.float64)
            y[t] += term
            S[t] += np.abs(term)
    return y, S


# --------------------------------------------------------------------------------------------
# the whole chain
# --------------------------------------------------------------------------------------------

def chain(x_bits, logits, gate_up, down, k: int, tile_m: int, alpha: float, limit: float):
    """One MoE layer from inputs only: route -> bucket -> gate_up (bias-seeded) -> SwiGLU-OAI ->
    bf16 h -> down (bias-seeded) -> slot-order combine ([fusion], [chain])."""
    T = x_bits.shape[0]
    E = gate_up["q"].shape[0]
    ids, w = route_topk(logits, k)
    mpad = mpad_max(T, k, E, tile_m)
    counts, basep, row_tok, pos = bucket(ids, E, tile_m, mpad)
    g, g_S = project(x_bits, row_tok, gate_up["q"], gate_up["s"], gate_up["bias"],
                     counts, basep, mpad)
    live = [r for _, r in live_rows(counts, basep)]
    h = np.zeros((mpad, g.shape[1] // 2), dtype=np.uint16)
    h[live] = bf16_round(swiglu_oai(g[live], alpha, limit))
    d, d_S = project(h, None, down["q"], down["s"], down["bias"], counts, basep, mpad)
    y, y_S = combine(d, pos, w)
    return {"ids": ids, "w": w, "mpad": mpad, "counts": counts, "basep": basep,
            "row_tok": row_tok, "pos": pos, "g": g, "g_S": g_S, "h": h, "d": d, "d_S": d_S,
            "y": y, "y_S": y_S}


def chain_mx8(x_bits, logits, gate_up, down, k: int, tile_m: int, alpha: float, limit: float):
    """The layer of `chain` with both projections on MXFP8 activations: the token rows x are
    quantized once (mx8_quantize) and gathered by the gate_up projection; the bf16 h rows are
    quantized after the SwiGLU-OAI (rows that are not live hold zeros and are never read) and
    feed the down projection. Routing, CSR, SwiGLU-OAI, the bf16 rounding of h and the combine
    are those of `chain`."""
    T = x_bits.shape[0]
    E = gate_up["q"].shape[0]
    ids, w = route_topk(logits, k)
    mpad = mpad_max(T, k, E, tile_m)
    counts, basep, row_tok, pos = bucket(ids, E, tile_m, mpad)
    xq, xs = mx8_quantize(x_bits)
    g, g_S = project_mx8(xq, xs, row_tok, gate_up["q"], gate_up["s"], gate_up["bias"],
                         counts, basep, mpad)
    live = [r for _, r in live_rows(counts, basep)]
    h = np.zeros((mpad, g.shape[1] // 2), dtype=np.uint16)
    h[live] = bf16_round(swiglu_oai(g[live], alpha, limit))
    hq, hs = mx8_quantize(h)
    d, d_S = project_mx8(hq, hs, None, down["q"], down["s"], down["bias"], counts, basep, mpad)
    y, y_S = combine(d, pos, w)
    return {"ids": ids, "w": w, "mpad": mpad, "counts": counts, "basep": basep,
            "row_tok": row_tok, "pos": pos, "xq": xq, "xs": xs, "g": g, "g_S": g_S, "h": h,
            "hq": hq, "hs": hs, "d": d, "d_S": d_S, "y": y, "y_S": y_S}
