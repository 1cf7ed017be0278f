"""Pins of the oracle's MXFP8 activation functions (E4M3 decode and encode, the MX block
conversion, the projection over MXFP8 rows) to facts outside the oracle: torch's own FP8 E4M3
conversion, closed forms of the OCP formats, brute force over the 127 finite magnitudes, and the
bf16 projection in the cases where the quantization loses nothing. No GPU is needed.
"""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_mixture_experts_route_amd import synth


def torch_e4m3_bits(v32):
    """torch's fp32 -> float8_e4m3fn conversion (round to nearest even; NaN past 464)."""
    return torch.from_numpy(np.asarray(v32, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_e4m3_decode_all_256_bytes_match_torch():
    # catches a wrong exponent bias, subnormal scale, sign, or a missing NaN code
    ref = torch.arange(256, dtype=torch.int64).to(torch.uint8).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()
    got = oracle.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_closed_forms():
    # the format's landmarks: largest finite 448, smallest normal 2^-6, smallest subnormal 2^-9
    d = oracle.e4m3_decode
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0 and oracle.E4M3_MAX == 448.0
    assert d(0x08) == 2.0 ** -6 and d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9
    assert d(0x38) == 1.0 and d(0x78) == 256.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))


def test_e4m3_encode_round_trips_every_finite_code():
    # catches an off-by-one in the quantum or a wrong code lookup
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes.astype(np.uint8))


def test_e4m3_encode_matches_torch_on_midpoints_and_random_values():
    # catches ties rounded away from even, truncation instead of rounding, wrong subnormal step
    mags = oracle.e4m3_decode(np.arange(127))
    mids = (mags[:-1] + mags[1:]) / 2                                   # exact in fp32
    around = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                             np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    rng = np.random.default_rng(7)
    rand = (rng.standard_normal(20000) * np.exp2(rng.integers(-14, 9, 20000))).astype(np.float32)
    rand = rand[np.abs(rand) < 460]
    v = np.concatenate([around.astype(np.float32), -around.astype(np.float32), rand])
    assert np.array_equal(oracle.e4m3_encode(v.astype(np.float64)), torch_e4m3_bits(v))


def test_e4m3_encode_saturates_and_keeps_the_sign_of_zero():
    # the MX conversion clamps to the largest finite value instead of making NaN
    e = oracle.e4m3_encode
    assert e([448.0, 449.0, 464.0, 465.0, 511.9, 1e30]).tolist() == [0x7E] * 6
    assert e([-465.0, -1e30]).tolist() == [0xFE, 0xFE]
    # 2^-10 is the tie between 0 and 2^-9: even code 0; 1.5 * 2^-10 rounds up
    assert e([0.0, -0.0, 2.0 ** -10, -2.0 ** -10, 1.5 * 2.0 ** -10]).tolist() == \
        [0x00, 0x80, 0x00, 0x80, 0x01]


def _bf16(v):
    return oracle.bf16_round(np.asarray(v, dtype=np.float64))


def test_mx8_quantize_hand_blocks():
    # scale = floor(log2(amax)) - 8 as an e8m0 byte; block max lands in [256, 512)
    rows = np.zeros((6, 32))
    rows[0, :] = 1.0                                   # amax 1 -> X = -8, 1 * 256 -> 0x78
    rows[1, 0], rows[1, 1] = 1.75, -0.5                # 448 exactly; -128 -> 0xF0
    rows[2, 0] = 1.9921875                             # largest bf16 below 2: 510 -> 448
    rows[3, 0] = -0.0                                  # all zero: smallest scale, sign kept
    rows[4, 0] = 2.0 ** -133                           # smallest bf16 subnormal: clamped scale
    rows[5, 0], rows[5, 1] = 3.0e38, 1.0e30            # near the top of the bf16 range
    q, s = oracle.mx8_quantize(_bf16(rows))
    assert s[:, 0].tolist() == [119, 119, 119, 0, 0, 127 + 127 - 8]
    assert q[0].tolist() == [0x78] * 32
    assert q[1, :2].tolist() == [0x7E, 0xF0]
    assert q[2, 0] == 0x7E
    assert q[3, 0] == 0x80 and not q[3, 1:].any()
    assert q[4, 0] == 0x08                             # 2^-133 * 2^127 = 2^-6
    x5 = oracle.bf16_to_f64(_bf16(rows[5, :2]))
    assert np.array_equal(oracle.mx8_dequant(q[5:6, :32], s[5:6, :1])[0, :2],
                          oracle.e4m3_decode(oracle.e4m3_encode(x5 / 2.0 ** 119)) * 2.0 ** 119)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mx8_quantize_scale_and_nearest_code_brute_force(seed):
    # every element gets the code of the nearest representable value (brute force over all 127
    # magnitudes), and an unclamped block's maximum scales into [256, 512)
    rng = np.random.default_rng(seed)
    rows = rng.standard_normal((8, 64)) * np.exp2(rng.integers(-30, 30, (8, 1)))
    rows[0, :32] *= 2.0 ** -120                        # a block whose scale clamps at -127
    bits = _bf16(rows)
    x = oracle.bf16_to_f64(bits)
    q, s = oracle.mx8_quantize(bits)
    mags = oracle.e4m3_decode(np.arange(127))
    for r in range(8):
        for b in range(2):
            blk = x[r, 32 * b:32 * b + 32]
            X = int(s[r, b]) - 127
            if X > -127:
                assert 256 <= np.abs(blk).max() / 2.0 ** X < 512
            for i in range(32):
                t = abs(blk[i]) / 2.0 ** X
                dist = np.abs(mags - t)
                best = np.flatnonzero(dist == dist.min())
                pick = best[0] if len(best) == 1 else best[best % 2 == 0][0]   # tie -> even
                assert q[r, 32 * b + i] & 0x7F == pick, (r, b, i)
                assert (q[r, 32 * b + i] >> 7) == int(np.signbit(blk[i]))


def test_project_mx8_equals_bf16_projection_when_quantization_is_lossless():
    # rows whose every block is X * (E4M3 values, one of them in [256, 448]) quantize exactly,
    # so the MXFP8 projection must equal the (pinned) bf16 projection bit for bit
    rng = np.random.default_rng(11)
    E, N, K, T, k, tile_m = 3, 16, 96, 6, 2, 4
    mags = oracle.e4m3_decode(np.arange(127))
    vals = rng.choice(mags, size=(T, K)) * rng.choice([-1.0, 1.0], size=(T, K))
    vals[:, ::32] = rng.choice(mags[(mags >= 256) & (mags <= 448)], size=(T, K // 32))
    vals *= np.repeat(np.exp2(rng.integers(-20, 5, (T, K // 32))), 32, axis=1)
    bits = _bf16(vals)
    assert np.array_equal(oracle.bf16_to_f64(bits), vals)
    xq, xs = oracle.mx8_quantize(bits)
    assert np.array_equal(oracle.mx8_dequant(xq, xs), vals)
    W = synth.random_mx4(3, E, N, K)
    ids, _ = oracle.route_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    mpad = oracle.mpad_max(T, k, E, tile_m)
    counts, basep, row_tok, _ = oracle.bucket(ids, E, tile_m, mpad)
    a, aS = oracle.project(bits, row_tok, W["q"], W["s"], W["bias"], counts, basep, mpad)
    b, bS = oracle.project_mx8(xq, xs, row_tok, W["q"], W["s"], W["bias"], counts, basep, mpad)
    assert np.array_equal(a, b, equal_nan=True) and np.array_equal(aS, bS, equal_nan=True)
    live = [r for _, r in oracle.live_rows(counts, basep)]
    samples = [(r, n) for r in live[:5] for n in (0, 7, 15)]
    v, vS = oracle.project_mx8_at(xq, xs, row_tok, W["q"], W["s"], W["bias"], counts, basep,
                                  samples)
    assert np.array_equal(v, np.array([a[r, n] for r, n in samples]))
