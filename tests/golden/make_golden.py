"""Writes tests/golden/tiny_chain.npz: the CPU oracle's outputs for the tiny MoE workload
(E=4, dim=ffn=64, top-2, T=8, tile_m=16, seed 0). Runs only the oracle and the seeded input
generator; the record guards the oracle and the generator against unintended change."""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from mxfp4_mixture_experts_route_amd import synth  # noqa: E402


def main():
    wl = synth.WORKLOADS["tiny"]
    tok = synth.tokens(wl)
    W = synth.layer_weights(wl)
    out = oracle.chain(tok["x"], tok["logits"], W["gate_up"], W["down"], wl.k, wl.tile_m,
                       synth.ALPHA, synth.LIMIT)
    keep = {k: out[k] for k in ("ids", "w", "counts", "basep", "row_tok", "pos", "g", "h", "d", "y")}
    np.savez_compressed(os.path.join(HERE, "tiny_chain.npz"), **keep)


if __name__ == "__main__":
    main()
