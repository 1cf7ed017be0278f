#!/usr/bin/env python3
"""Benchmark of the routed MXFP4 MoE chain on one MI355X (gfx950).

A step is one pass of the whole chain (route -> bucket -> gate_up + SwiGLU-OAI -> down ->
combine) over one batch. The headline workload is gpt-oss-20b-shaped decode: E=32 experts,
dim = ffn = 2880, top-4, one token, through 24 distinct seeded MoE layers (10.15 GB of MXFP4
experts resident in HBM, 1.27 GB touched per step, far more than the 256 MB last-level cache), so a
step is one decode token through the model's 24 MoE layers, replayed as one HIP graph. Each layer
runs as mx4_moe_decode (the chain fused into two launches); the five-call chain (route, bucket,
GEMV, GEMV, combine) is timed beside it, and moe_router (router projection + top-k + CSR in one
launch) on the same tokens.

Prints ONE JSON line. `value` = decode tokens/s through the 24-layer stack. The same line also
carries the dominant kernel's roofline, the decode weight GB/s of the two MXFP4 projections, the
pp512 prefill expert-GEMM TFLOP/s (gpt-oss-20b shape, T=512, bf16 MFMA, and beside it the same
layers with MXFP8 activations on the MX-scaled MFMA), and the CPU oracle timed on a bounded sample
of the decode workload on the host cores. Kernel durations come from the
library's kernel timing (moe_timing_arm: HIP events the runtime stamps at each kernel's own start
and end, on the stream it runs on), the interval a rocprofv3 kernel trace reports.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-prefill]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_DENSE_TFLOPS = 2500.0      # MI355X bf16 dense MFMA
FP8_DENSE_TFLOPS = 5000.0       # MI355X fp8 dense MFMA (the rate of an fp4 x fp8 MX product)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--kernel-reps", type=int, default=4, help="passes of per-kernel timing")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=12.0)
    p.add_argument("--counter-pass", action="store_true",
                   help="run only what the hardware-counter passes measure: a plain copy kernel of "
                        "known size, then the fused decode of 8 layers twice (no timing, no JSON)")
    p.add_argument("--counter-pass-prefill", action="store_true",
                   help="the same for the pp512 expert GEMMs: the copy kernel, then the pp512 chain "
                        "over its layers twice with bf16 and twice with MXFP8 activations")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Layer:
    """One MoE layer resident on the GPU with preallocated intermediates (graph-capturable)."""

    def __init__(self, moe, synth, torch, wl, l, kernel, W=None, tok=None):
        self.moe, self.wl = moe, wl
        tok = tok if tok is not None else synth.tokens(wl, l)
        W = W if W is not None else synth.layer_weights(wl, l)
        dev = "cuda"
        self.x = torch.from_numpy(tok["x"].view("int16")).to(dev).view(torch.bfloat16)
        self.logits = torch.from_numpy(tok["logits"]).to(dev)
        self.GU = moe.MX4Experts.from_numpy(W["gate_up"], dev)
        self.DN = moe.MX4Experts.from_numpy(W["down"], dev)
        T, E, k, D, F = wl.T, wl.E, wl.k, wl.dim, wl.ffn
        self.mpad = moe.moe_mpad_max(T, k, E, wl.tile_m)
        i32, f32 = torch.int32, torch.float32
        self.ids = torch.empty((T, k), dtype=i32, device=dev)
        self.w = torch.empty((T, k), dtype=f32, device=dev)
        self.csr = (torch.empty(E, dtype=i32, device=dev), torch.empty(E + 1, dtype=i32, device=dev),
                    torch.empty(self.mpad, dtype=i32, device=dev),
                    torch.empty((T, k), dtype=i32, device=dev))
        self.h = torch.empty((self.mpad, F), dtype=torch.bfloat16, device=dev)
        self.d = torch.empty((self.mpad, D), dtype=f32, device=dev)
        self.y = torch.empty((T, D), dtype=f32, device=dev)
        self.proj = moe.mx4_moe_gemm if kernel == "gemm" else moe.mx4_moe_gemv

    def route_bucket(self):
        m, wl = self.moe, self.wl
        m.moe_route_topk(self.logits, wl.k, ids=self.ids, w=self.w)
        m.moe_bucket(self.ids, wl.E, wl.tile_m, self.mpad, out=self.csr)

    def gate_up(self):
        c = self.csr
        self.proj(self.x, c[2], self.GU, c[0], c[1], self.wl.tile_m, self.mpad,
                  self.moe.MOE_ACT_SWIGLU_OAI, 1.702, 7.0, out=self.h)

    def down(self):
        c = self.csr
        self.proj(self.h, None, self.DN, c[0], c[1], self.wl.tile_m, self.mpad,
                  self.moe.MOE_ACT_NONE, 1.702, 7.0, out=self.d)

    def combine(self):
        self.moe.moe_combine(self.d, self.csr[3], self.w, out=self.y)

    def chain(self):
        self.route_bucket()
        self.gate_up()
        self.down()
        self.combine()

    def alloc_mx8(self, torch):
        """MXFP8 copies of x and h for chain_mx8."""
        u8, sp, wl = torch.uint8, self.moe.scale_row_bytes, self.wl
        self.xq = torch.empty((wl.T, wl.dim), dtype=u8, device="cuda")
        self.xs = torch.empty((wl.T, sp(wl.dim)), dtype=u8, device="cuda")
        self.hq = torch.empty((self.mpad, wl.ffn), dtype=u8, device="cuda")
        self.hs = torch.empty((self.mpad, sp(wl.ffn)), dtype=u8, device="cuda")

    def chain_mx8(self):
        """The chain with MXFP8 activations: route, bucket, quantize x, gate_up (MX MFMA, h
        written as MXFP8 rows by its epilogue), down (MX MFMA), combine (6 launches)."""
        m, wl, c = self.moe, self.wl, self.csr
        self.route_bucket()
        m.mx8_quantize(self.x, out=(self.xq, self.xs))
        m.mx4_moe_gemm_mx8(self.xq, self.xs, c[2], self.GU, c[0], c[1], wl.tile_m, self.mpad,
                           m.MOE_ACT_SWIGLU_OAI_MX8, 1.702, 7.0, out=self.hq,
                           out_scale=self.hs)
        m.mx4_moe_gemm_mx8(self.hq, self.hs, None, self.DN, c[0], c[1], wl.tile_m, self.mpad,
                           m.MOE_ACT_NONE, 1.702, 7.0, out=self.d)
        self.combine()

    def decode_persistent(self, ws):
        """The chain as mx4_moe_decode_persistent (one launch)."""
        c = self.csr
        self.moe.mx4_moe_decode_persistent(self.logits, self.x, self.GU, self.DN, self.wl.k, ws,
                                           1.702, 7.0,
                                           out={"ids": self.ids, "w": self.w, "counts": c[0],
                                                "basep": c[1], "row_tok": c[2], "pos": c[3],
                                                "h": self.h, "y": self.y})

    def decode(self):
        """The chain as mx4_moe_decode (two launches; h in routed-row order, T*k rows)."""
        c = self.csr
        self.moe.mx4_moe_decode(self.logits, self.x, self.GU, self.DN, self.wl.k, 1.702, 7.0,
                                out={"ids": self.ids, "w": self.w, "counts": c[0], "basep": c[1],
                                     "row_tok": c[2], "pos": c[3], "h": self.h, "y": self.y})


def build_layers(moe, synth, torch, wl, kernel, n_layers):
    out = []

    def gen(l):
        return l, synth.layer_weights(wl, l), synth.tokens(wl, l)

    with ThreadPoolExecutor(max_workers=8) as ex:
        for l, W, tok in ex.map(gen, range(n_layers)):
            out.append(Layer(moe, synth, torch, wl, l, kernel, W=W, tok=tok))
            del W, tok
    torch.cuda.synchronize()
    return out


def sleep_cycles_for(torch, ms):
    """Cycle count for torch.cuda._sleep lasting about `ms` (calibrated once), or 0 if absent."""
    if not hasattr(torch.cuda, "_sleep"):
        return 0
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    s.record()
    torch.cuda._sleep(1_000_000)
    e.record()
    torch.cuda.synchronize()
    per_ms = 1_000_000 / max(s.elapsed_time(e), 1e-3)
    return int(per_ms * ms)


def graph_time(torch, fn, steps, warmup):
    """Capture fn() as one HIP graph, replay warmup + timed steps; seconds for the timed ones."""
    fn()                                  # eager first call (one-time library set-up)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0, g


def kernel_times_us(moe, torch, layers, call, launches, reps, sleep_cycles):
    """Average kernel duration (us) of each of the `launches` kernels that call(L) makes per
    layer, from the library's kernel timing (events stamped at each kernel's own start and end).
    Layers are queued back to back behind a sleep kernel, in batches that fit MOE_TIMING_MAX."""
    per_batch = max(1, 64 // launches)
    sums = [0.0] * launches
    n = 0
    for _ in range(reps):
        for b0 in range(0, len(layers), per_batch):
            batch = layers[b0:b0 + per_batch]
            torch.cuda.synchronize()
            if sleep_cycles:
                torch.cuda._sleep(sleep_cycles)
            moe.moe_timing_arm(len(batch) * launches)
            for L in batch:
                call(L)
            ms = moe.moe_timing_read(len(batch) * launches)
            moe.moe_timing_arm(0)
            for i in range(len(batch)):
                for j in range(launches):
                    sums[j] += ms[i * launches + j]
            n += len(batch)
    return [1000.0 * v / n for v in sums]


def router_us(moe, torch, layers, wl, reps, sleep_cycles):
    """Kernel time of moe_router (router projection + top-k + CSR, one launch) on the layers'
    x with a seeded bf16 router [E][D] and bias, writing into the layers' routing buffers."""
    g = torch.Generator(device="cpu").manual_seed(99)
    wr = (torch.randn((wl.E, wl.dim), generator=g) / wl.dim ** 0.5).to(torch.bfloat16).cuda()
    br = (torch.randn(wl.E, generator=g) * 0.1).cuda()
    sync = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call(L):
        c = L.csr
        moe.moe_router(L.x, wr, br, wl.k, wl.tile_m, sync, mpad_max=L.mpad, want_logits=False,
                       out={"ids": L.ids, "w": L.w, "counts": c[0], "basep": c[1],
                            "row_tok": c[2], "pos": c[3]})
    return kernel_times_us(moe, torch, layers, call, 1, reps, sleep_cycles)[0]


def touched_experts(torch, layers):
    return [int(torch.unique(L.ids).numel()) for L in layers]


def cpu_baseline(synth, wl, budget_s):
    """The CPU oracle (as it stands) on one decode token per layer, as many layers as fit in the
    budget, on one host thread; scaled to the 24-layer stack's tokens/s."""
    import oracle
    from threadpoolctl import threadpool_limits
    times = []
    with threadpool_limits(limits=1):
        t_all = time.perf_counter()
        for l in range(wl.layers):
            tok = synth.tokens(wl, l)
            W = synth.layer_weights(wl, l)
            t0 = time.perf_counter()
            oracle.chain(tok["x"], tok["logits"], W["gate_up"], W["down"], wl.k, wl.tile_m,
                         synth.ALPHA, synth.LIMIT)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_all > budget_s:
                break
    per_layer = sum(times) / len(times)
    return {"value": round(wl.T / (per_layer * wl.layers), 4), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"oracle.chain (float64 numpy, 1 thread) on 1 token through layers 0..{len(times) - 1} "
                      f"of the 24-layer decode workload; {per_layer * 1e3:.0f} ms per layer, "
                      f"scaled to 24 layers"}


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "decode_gate_up_kernel_traffic_decode_t1.md")
TRAFFIC_SOURCES = ("decode.hip", "gemv_core.hpp", "route_core.hpp", "common.hpp")


def kernel_source_hash():
    """sha256 over the sources of the fused decode kernels (any change invalidates counters)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "mxfp4_mixture_experts_route_amd", "csrc")
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the fused gate_up kernel from the committed counter summary, or
    None when there is none or the kernel's sources changed since the counters were taken."""
    try:
        fields = dict(line.strip("` \n").split("=", 1) for line in open(TRAFFIC_FILE)
                      if line.startswith("`") and "=" in line)
    except OSError:
        return None
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    return int(float(fields["traffic_bytes_per_launch"]))


def counter_pass(moe, synth, torch):
    """Workload of the rocprofv3 --pmc passes: a copy kernel of 64 MiB (read 64 MiB, write
    64 MiB) three times for the counters' scale, then mx4_moe_decode over 8 layers, twice."""
    copy_kernel_pass(torch)
    wl = synth.WORKLOADS["decode_t1"]
    layers = build_layers(moe, synth, torch, wl, "gemv", 8)
    for _ in range(2):
        for L in layers:
            L.decode()
    torch.cuda.synchronize()
    log("counter pass done")


def copy_kernel_pass(torch):
    """A plain copy of known size (reads 64 MiB, writes 64 MiB) three times: the counters' scale."""
    src = torch.ones(16 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()


def counter_pass_prefill(moe, synth, torch):
    """Workload of the rocprofv3 --pmc passes for the pp512 GEMMs: the copy kernel, then every
    layer's chain twice with bf16 activations and twice with MXFP8 activations (4 layers, 1.7 GB
    of experts, so no layer's weights are cache-resident from the previous one)."""
    copy_kernel_pass(torch)
    pw = synth.WORKLOADS["prefill_pp512"]
    players = build_layers(moe, synth, torch, pw, "gemm", pw.layers)
    for _ in range(2):
        for L in players:
            L.chain()
    torch.cuda.synchronize()
    for L in players:
        L.alloc_mx8(torch)
    for _ in range(2):
        for L in players:
            L.chain_mx8()
    torch.cuda.synchronize()
    log("prefill counter pass done")


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); expert parallelism "
              "across GPUs is not implemented.", file=sys.stderr)
        sys.exit(2)
    import numpy as np  # noqa: F401
    import torch
    from mxfp4_mixture_experts_route_amd import _lib as moe
    from mxfp4_mixture_experts_route_amd import synth
    moe.lib()   # fail loudly if the HIP library is missing
    torch.cuda.init()
    if args.counter_pass:
        counter_pass(moe, synth, torch)
        return
    if args.counter_pass_prefill:
        counter_pass_prefill(moe, synth, torch)
        return
    sleep_cycles = sleep_cycles_for(torch, 20.0)

    # ---------------- headline: decode, T=1, 24 MoE layers ----------------
    wl = synth.WORKLOADS["decode_t1"]
    log(f"building {wl.layers} layers of {wl.desc}")
    layers = build_layers(moe, synth, torch, wl, "gemv", wl.layers)
    log(f"timing {args.steps} graph-replayed steps after {args.warmup} warmup (fused decode)")
    secs, _ = graph_time(torch, lambda: [L.decode() for L in layers], args.steps, args.warmup)
    ms_per_step = 1000.0 * secs / args.steps
    tokens_per_s = wl.T * args.steps / secs
    log("the same steps as the five-call chain")
    secs5, _ = graph_time(torch, lambda: [L.chain() for L in layers], args.steps, args.warmup)

    log("kernel timing")
    fused_us = kernel_times_us(moe, torch, layers, lambda L: L.decode(), 2, args.kernel_reps,
                               sleep_cycles)
    chain_us = kernel_times_us(moe, torch, layers, lambda L: L.chain(), 5, args.kernel_reps,
                               sleep_cycles)
    n_touch = touched_experts(torch, layers)
    decode_router_us = router_us(moe, torch, layers, wl, args.kernel_reps, sleep_cycles)
    per_expert_gu = 2 * wl.ffn * wl.dim * 17 // 32          # nibbles + scales, bytes
    per_expert_dn = wl.dim * wl.ffn * 17 // 32
    avg_touch = sum(n_touch) / len(n_touch)
    gu_bytes = avg_touch * per_expert_gu
    dn_bytes = avg_touch * per_expert_dn
    gu_gbps = gu_bytes / (fused_us[0] * 1e3)
    fused_gbps = (gu_bytes + dn_bytes) / ((fused_us[0] + fused_us[1]) * 1e3)
    gemv_gbps = (gu_bytes + dn_bytes) / ((chain_us[2] + chain_us[3]) * 1e3)

    result = {
        "metric": "MoE chain tokens/s; decode mx4 weight GB/s; pp512 expert GEMM TFLOP/s (1 GPU)",
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gpt-oss-20b-shaped decode, T=1, 24 distinct MoE layers per step",
                   "E": wl.E, "dim": wl.dim, "ffn": wl.ffn, "k": wl.k, "T": wl.T,
                   "layers": wl.layers, "weights": "mxfp4", "accumulate": "f32",
                   "chain": "mx4_moe_decode (2 launches per layer)", "graph": "hip graph replay"},
        "roofline": {"kernel": "decode_gate_up_kernel (routing + gate_up + SwiGLU-OAI)",
                     "bound": "hbm", "achieved": round(gu_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gu_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(),
                     "bytes_per_launch": int(gu_bytes), "avg_launch_us": round(fused_us[0], 3)},
        "decode": {"fused": {"gate_up_kernel_us": round(fused_us[0], 3),
                             "down_combine_kernel_us": round(fused_us[1], 3),
                             "weight_GBps": round(fused_gbps, 1),
                             "frac_hbm_peak": round(fused_gbps / HBM_PEAK_GBPS, 4),
                             "per_layer_us": round(ms_per_step * 1000.0 / wl.layers, 3)},
                   "five_call_chain": {"tokens_per_s": round(wl.T * args.steps / secs5, 2),
                                       "per_layer_us": round(1e6 * secs5 / (args.steps * wl.layers), 3),
                                       "route_us": round(chain_us[0], 3),
                                       "bucket_us": round(chain_us[1], 3),
                                       "gemv_gate_up_us": round(chain_us[2], 3),
                                       "gemv_down_us": round(chain_us[3], 3),
                                       "combine_us": round(chain_us[4], 3),
                                       "gemv_weight_GBps": round(gemv_gbps, 1)},
                   "touched_experts_per_layer": avg_touch,
                   "router_us": round(decode_router_us, 3)},
    }
    del layers
    torch.cuda.empty_cache()

    # ---------------- pp512 prefill expert GEMM ----------------
    if not args.no_prefill:
        pw = synth.WORKLOADS["prefill_pp512"]
        log(f"building {pw.layers} layers of {pw.desc}")
        players = build_layers(moe, synth, torch, pw, "gemm", pw.layers)
        psecs, _ = graph_time(torch, lambda: [L.chain() for L in players], max(5, args.steps // 5),
                              args.warmup)
        p_steps = max(5, args.steps // 5)
        pkt = kernel_times_us(moe, torch, players, lambda L: L.chain(), 5, args.kernel_reps,
                              sleep_cycles)
        pkt = {"gate_up": pkt[2], "down": pkt[3]}
        R = pw.T * pw.k
        flops = 2.0 * R * pw.dim * 3 * pw.ffn
        tflops = flops / ((pkt["gate_up"] + pkt["down"]) * 1e-6) / 1e12
        result["prefill_pp512"] = {
            "expert_gemm_TFLOPs": round(tflops, 1),
            "frac_bf16_peak": round(tflops / BF16_DENSE_TFLOPS, 4),
            "gate_up_us": round(pkt["gate_up"], 2), "down_us": round(pkt["down"], 2),
            "chain_tokens_per_s": round(pw.T * pw.layers * p_steps / psecs, 1),
            "per_layer_chain_us": round(1e6 * psecs / (p_steps * pw.layers), 2),
            "flops_per_layer": flops,
        }
        log("pp512 with MXFP8 activations (MX-scaled MFMA)")
        for L in players:
            L.alloc_mx8(torch)
        msecs, _ = graph_time(torch, lambda: [L.chain_mx8() for L in players], p_steps,
                              args.warmup)
        mkt = kernel_times_us(moe, torch, players, lambda L: L.chain_mx8(), 6, args.kernel_reps,
                              sleep_cycles)
        mx_tflops = flops / ((mkt[3] + mkt[4]) * 1e-6) / 1e12
        result["prefill_pp512"]["mx8"] = {
            "activations": "MXFP8 (E4M3 + e8m0 per 32), v_mfma_scale_f32_16x16x128_f8f6f4",
            "expert_gemm_TFLOPs": round(mx_tflops, 1),
            "frac_fp8_peak": round(mx_tflops / FP8_DENSE_TFLOPS, 4),
            "gate_up_us": round(mkt[3], 2), "down_us": round(mkt[4], 2),
            "quantize_x_us": round(mkt[2], 2),
            "h_quantized_in": "the gate_up epilogue (MOE_ACT_SWIGLU_OAI_MX8)",
            "chain_tokens_per_s": round(pw.T * pw.layers * p_steps / msecs, 1),
            "per_layer_chain_us": round(1e6 * msecs / (p_steps * pw.layers), 2),
        }
        result["prefill_pp512"]["router_us"] = round(
            router_us(moe, torch, players, pw, args.kernel_reps, sleep_cycles), 2)
        del players
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(synth, wl, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
