"""Seeded synthetic inputs for the routed MXFP4 expert chain.

This module only draws random numbers in the shapes and distributions of the gpt-oss MoE
workloads; it contains none of the chain's arithmetic (no decoding, routing, bucketing or
projection). Both the HIP path's tests/bench and the CPU oracle's tests take their inputs
from here, so the two sides share inputs and never code.

Distributions (every workload):
  x        bf16 [T][dim]: standard normal draws, rounded to bf16 (round-to-nearest-even)
  logits   f32  [T][E]:   normal draws with the workload's standard deviation, plus the
                           workload's structure (a hot expert, or experts that get no token)
  weights  MXFP4: nibble bytes uniform over [0, 256) (so all 16 e2m1 codes appear), e8m0
           scale bytes uniform over [118, 124], biases f32 normal with std 0.02
  gate_up  q [E][2*ffn][dim/2], s [E][2*ffn][dim/32], b [E][2*ffn]
  down     q [E][dim][ffn/2],   s [E][dim][ffn/32],   b [E][dim]

Seeds: a workload's layer l draws from numpy's PCG64 seeded with (seed_base + l, stream) where
stream separates the arrays, so any one array can be regenerated alone.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ALPHA = 1.702   # SwiGLU-OAI sigmoid slope of gpt-oss
LIMIT = 7.0     # SwiGLU-OAI clamp of gpt-oss

# array stream ids (independent PCG64 streams per array)
_S_X, _S_LOGITS, _S_DEAD = 1, 2, 3
_S_GU_Q, _S_GU_S, _S_GU_B = 11, 12, 13
_S_DN_Q, _S_DN_S, _S_DN_B = 21, 22, 23

SCALE_LO, SCALE_HI = 118, 124   # e8m0 bytes: 2^-9 .. 2^-3
BIAS_STD = 0.02


@dataclass(frozen=True)
class Workload:
    name: str
    E: int
    dim: int
    ffn: int
    k: int
    T: int
    tile_m: int
    layers: int = 1
    seed_base: int = 0
    logit_std: float = 1.0
    hot_expert: int | None = None   # this expert's logit column gets +hot_bias
    hot_bias: float = 0.0
    n_dead: int = 0                 # this many seeded experts get logit -30 (receive no token)
    desc: str = field(default="", compare=False)

    @property
    def R(self) -> int:
        return self.T * self.k


# The five MoE workloads of the gpt-oss family at their real shapes.
WORKLOADS = {
    "tiny": Workload(
        "tiny", E=4, dim=64, ffn=64, k=2, T=8, tile_m=16, layers=1, seed_base=0,
        desc="tiny MoE layer, E=4, dim=ffn=64, top-2, T=8"),
    "decode_t1": Workload(
        "decode_t1", E=32, dim=2880, ffn=2880, k=4, T=1, tile_m=1, layers=24, seed_base=1000,
        desc="gpt-oss-20b-shaped decode, T=1, 24 distinct MoE layers"),
    "decode_t64": Workload(
        "decode_t64", E=32, dim=2880, ffn=2880, k=4, T=64, tile_m=16, layers=4, seed_base=2000,
        hot_expert=0, hot_bias=2.0,
        desc="gpt-oss-20b-shaped batched decode, T=64, expert 0 biased +2"),
    "prefill_pp512": Workload(
        "prefill_pp512", E=32, dim=2880, ffn=2880, k=4, T=512, tile_m=16, layers=4, seed_base=3000,
        desc="gpt-oss-20b-shaped prefill pp512, T=512"),
    "prefill_120b_t2048": Workload(
        "prefill_120b_t2048", E=128, dim=2880, ffn=2880, k=4, T=2048, tile_m=16, layers=2,
        seed_base=4000, logit_std=1.5, n_dead=8,
        desc="gpt-oss-120b-shaped prefill, T=2048, 8 experts receive no token"),
}


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([seed, stream]))


def round_f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float32 values, round-to-nearest-even (torch's conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact: the bf16 bits become the high half)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def tokens(wl: Workload, layer: int = 0) -> dict:
    """Activations x (bf16 bits) and router logits (f32) for one layer of the workload."""
    seed = wl.seed_base + layer
    x = round_f32_to_bf16_bits(_rng(seed, _S_X).standard_normal((wl.T, wl.dim), dtype=np.float32))
    logits = (_rng(seed, _S_LOGITS).standard_normal((wl.T, wl.E), dtype=np.float32)
              * np.float32(wl.logit_std))
    if wl.hot_expert is not None:
        logits[:, wl.hot_expert] += np.float32(wl.hot_bias)
    dead = np.zeros(0, dtype=np.int64)
    if wl.n_dead:
        dead = np.sort(_rng(seed, _S_DEAD).choice(wl.E, size=wl.n_dead, replace=False))
        logits[:, dead] = np.float32(-30.0)
    return {"x": x, "logits": np.ascontiguousarray(logits, dtype=np.float32), "dead": dead}


def _mx4(seed: int, sq: int, ss: int, sb: int, E: int, N: int, K: int) -> dict:
    q = np.frombuffer(_rng(seed, sq).bytes(E * N * (K // 2)), dtype=np.uint8).reshape(E, N, K // 2)
    s = _rng(seed, ss).integers(SCALE_LO, SCALE_HI + 1, size=(E, N, K // 32), dtype=np.uint8)
    b = (_rng(seed, sb).standard_normal((E, N), dtype=np.float32) * np.float32(BIAS_STD))
    return {"q": q, "s": s, "bias": b.astype(np.float32)}


def layer_weights(wl: Workload, layer: int = 0) -> dict:
    """MXFP4 expert weights of one layer: {'gate_up': {q,s,bias}, 'down': {q,s,bias}}."""
    seed = wl.seed_base + layer
    return {
        "gate_up": _mx4(seed, _S_GU_Q, _S_GU_S, _S_GU_B, wl.E, 2 * wl.ffn, wl.dim),
        "down": _mx4(seed, _S_DN_Q, _S_DN_S, _S_DN_B, wl.E, wl.dim, wl.ffn),
    }


def random_mx4(seed: int, E: int, N: int, K: int, scale_lo: int = SCALE_LO,
               scale_hi: int = SCALE_HI, bias_std: float | None = BIAS_STD) -> dict:
    """An MXFP4 expert stack of arbitrary shape with the workload distributions (test sizes)."""
    g = _rng(seed, 101)
    q = np.frombuffer(g.bytes(E * N * (K // 2)), dtype=np.uint8).reshape(E, N, K // 2)
    s = g.integers(scale_lo, scale_hi + 1, size=(E, N, K // 32), dtype=np.uint8)
    b = None if bias_std is None else (g.standard_normal((E, N), dtype=np.float32)
                                       * np.float32(bias_std)).astype(np.float32)
    return {"q": q, "s": s, "bias": b}


def random_bf16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns of normal draws (test sizes)."""
    v = _rng(seed, 102).standard_normal(shape, dtype=np.float32) * np.float32(std)
    return round_f32_to_bf16_bits(v)


def random_logits(seed: int, T: int, E: int, std: float = 1.0) -> np.ndarray:
    return (_rng(seed, 103).standard_normal((T, E), dtype=np.float32) * np.float32(std))


def random_ids(seed: int, T: int, k: int, E: int, skew: float = 0.0) -> np.ndarray:
    """k distinct expert ids per token (optionally skewed toward low ids), for CSR tests."""
    g = _rng(seed, 104)
    p = np.exp(-skew * np.arange(E) / max(E, 1))
    p /= p.sum()
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        out[t] = g.choice(E, size=k, replace=False, p=p)
    return out
