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

The same JSON line carries the other gpt-oss workloads, each timed the same way (graph-replayed
chain, per-kernel times): batched decode T=64 with a hot expert (weight GB/s), prefill pp512 and
the 120b-shaped T=2048 layer with dead experts (expert-GEMM TFLOP/s, bf16 and MXFP8 activations);
the attained peaks of this GPU (a plain streaming read at three sizes, a bf16 MFMA loop); and the
CPU oracle timed on bounded samples on the host cores (one thread and all of them).

Kernel durations come from the library's kernel timing (moe_timing_arm: HIP events the runtime
stamps at each kernel's own start and end, on the stream it runs on), the interval a rocprofv3
kernel trace reports. Those timing passes are bracketed by roctxProfilerResume/Pause, so
`rocprofv3 --kernel-trace --stats --selected-regions -- python3 bench.py ...` traces exactly the
dispatches whose durations the line reports.

Prints ONE JSON line. `value` = decode tokens/s through the 24-layer stack.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--parts decode,t64,pp512,120b,peaks,cpu]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time
from concurrent.futures import ThreadPoolExecutor

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_DENSE_TFLOPS = 2500.0      # MI355X bf16 dense MFMA
FP8_DENSE_TFLOPS = 5000.0       # MI355X fp8 dense MFMA (the rate of an fp4 x fp8 MX product)
PARTS = ("decode", "t64", "pp512", "120b", "peaks", "cpu")
ALPHA, LIMIT = 1.702, 7.0


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--kernel-reps", type=int, default=4, help="passes of per-kernel timing")
    p.add_argument("--parts", default=",".join(PARTS),
                   help="comma-separated subset of " + ",".join(PARTS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true", help="skip pp512 and 120b")
    p.add_argument("--cpu-budget-s", type=float, default=8.0,
                   help="wall-time budget of each CPU oracle sample")
    p.add_argument("--counter-pass", nargs="?", const="decode_t1", default=None,
                   metavar="WORKLOAD",
                   help="run only what the hardware-counter passes measure: a plain copy kernel "
                        "of known size, then the workload's chain twice (no timing, no JSON)")
    p.add_argument("--counter-pass-prefill", action="store_true",
                   help="--counter-pass prefill_pp512, with MXFP8 activations as well")
    args = p.parse_args(argv)
    parts = [s for s in args.parts.split(",") if s]
    bad = [s for s in parts if s not in PARTS]
    if bad:
        p.error(f"unknown parts {bad}")
    if args.no_cpu_baseline and "cpu" in parts:
        parts.remove("cpu")
    if args.no_prefill:
        parts = [s for s in parts if s not in ("pp512", "120b")]
    args.parts = parts
    return args


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Roctx:
    """roctxProfilerResume/Pause around the timing passes (no-ops where the library is absent):
    under `rocprofv3 --selected-regions` only those regions are traced."""

    def __init__(self):
        self.lib = None
        for name in ("librocprofiler-sdk-roctx.so.1", "/opt/rocm/lib/librocprofiler-sdk-roctx.so.1"):
            try:
                self.lib = ctypes.CDLL(name)
                self.lib.roctxProfilerResume.argtypes = [ctypes.c_uint64]
                self.lib.roctxProfilerPause.argtypes = [ctypes.c_uint64]
                break
            except (OSError, AttributeError):
                self.lib = None

    def __enter__(self):
        if self.lib:
            self.lib.roctxProfilerResume(0)
        return self

    def __exit__(self, *exc):
        if self.lib:
            self.lib.roctxProfilerPause(0)
        return False


ROCTX = None


class Marked:
    """A timing region, marked in kernel traces: a one-workgroup moe_probe_read of 16 bytes
    right before and right after it (on the current stream), inside a roctx resume/pause pair.
    `bench.py --trace-summary` takes the dispatches between such markers."""

    def __init__(self, moe, torch):
        self.moe = moe
        self.buf = torch.zeros(4, dtype=torch.int32, device="cuda")
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def mark(self):
        self.moe.moe_probe_read(self.buf, 1, sink=self.sink)

    def __enter__(self):
        ROCTX.__enter__()
        self.mark()
        return self

    def __exit__(self, *exc):
        self.mark()
        ROCTX.__exit__(*exc)
        return False


MARK = None


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
        self.set_kernel(kernel)

    def set_kernel(self, kernel):
        self.proj = self.moe.mx4_moe_gemm if kernel == "gemm" else self.moe.mx4_moe_gemv

    def route_bucket(self):
        m, wl = self.moe, self.wl
        m.moe_route_topk(self.logits, wl.k, ids=self.ids, w=self.w)
        m.moe_bucket(self.ids, wl.E, wl.tile_m, self.mpad, out=self.csr)

    def gate_up(self):
        c = self.csr
        self.proj(self.x, c[2], self.GU, c[0], c[1], self.wl.tile_m, self.mpad,
                  self.moe.MOE_ACT_SWIGLU_OAI, ALPHA, LIMIT, out=self.h)

    def down(self):
        c = self.csr
        self.proj(self.h, None, self.DN, c[0], c[1], self.wl.tile_m, self.mpad,
                  self.moe.MOE_ACT_NONE, ALPHA, LIMIT, out=self.d)

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
                           m.MOE_ACT_SWIGLU_OAI_MX8, ALPHA, LIMIT, out=self.hq,
                           out_scale=self.hs)
        m.mx4_moe_gemm_mx8(self.hq, self.hs, None, self.DN, c[0], c[1], wl.tile_m, self.mpad,
                           m.MOE_ACT_NONE, ALPHA, LIMIT, out=self.d)
        self.combine()

    def decode_persistent(self, ws):
        """The chain as mx4_moe_decode_persistent (one launch)."""
        c = self.csr
        self.moe.mx4_moe_decode_persistent(self.logits, self.x, self.GU, self.DN, self.wl.k, ws,
                                           ALPHA, LIMIT,
                                           out={"ids": self.ids, "w": self.w, "counts": c[0],
                                                "basep": c[1], "row_tok": c[2], "pos": c[3],
                                                "h": self.h, "y": self.y})

    def decode(self):
        """The chain as mx4_moe_decode (two launches; h in routed-row order, T*k rows)."""
        c = self.csr
        self.moe.mx4_moe_decode(self.logits, self.x, self.GU, self.DN, self.wl.k, ALPHA, LIMIT,
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
    Layers are queued back to back behind a sleep kernel, in batches that fit MOE_TIMING_MAX.
    One untimed pass first (first-call set-up); the timed passes run inside a roctx region."""
    per_batch = max(1, 64 // launches)
    for L in layers:
        call(L)
    torch.cuda.synchronize()
    sums = [0.0] * launches
    n = 0
    with MARK:
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
    ws = torch.zeros(moe.MOE_ROUTER_WS_WORDS, dtype=torch.int32, device="cuda")

    def call(L):
        c = L.csr
        moe.moe_router(L.x, wr, br, wl.k, wl.tile_m, ws, mpad_max=L.mpad, want_logits=False,
                       out={"ids": L.ids, "w": L.w, "counts": c[0], "basep": c[1],
                            "row_tok": c[2], "pos": c[3]})
    return kernel_times_us(moe, torch, layers, call, 1, reps, sleep_cycles)[0]


def touched_experts(torch, layers):
    return [int(torch.unique(L.ids).numel()) for L in layers]


def expert_bytes(wl):
    """MXFP4 bytes (nibbles + scales) of one expert's gate_up and down projections."""
    return 2 * wl.ffn * wl.dim * 17 // 32, wl.dim * wl.ffn * 17 // 32


def chain_flops(wl):
    """Algorithmic flops of the two projections on the live routed rows."""
    return 2.0 * wl.T * wl.k * wl.dim * 3 * wl.ffn


def r1(v, nd=2):
    return None if v is None else round(v, nd)


# ------------------------------------------------------------------------------------------
# workloads
# ------------------------------------------------------------------------------------------

def bench_decode(moe, synth, torch, args, sleep_cycles):
    wl = synth.WORKLOADS["decode_t1"]
    log(f"building {wl.layers} layers of {wl.desc}")
    layers = build_layers(moe, synth, torch, wl, "gemv", wl.layers)
    log(f"timing {args.steps} graph-replayed steps after {args.warmup} warmup (fused decode)")
    secs, _ = graph_time(torch, lambda: [L.decode() for L in layers], args.steps, args.warmup)
    log("the same steps as the five-call chain")
    secs5, _ = graph_time(torch, lambda: [L.chain() for L in layers], args.steps, args.warmup)
    log("kernel timing")
    fused_us = kernel_times_us(moe, torch, layers, lambda L: L.decode(), 2, args.kernel_reps,
                               sleep_cycles)
    chain_us = kernel_times_us(moe, torch, layers, lambda L: L.chain(), 5, args.kernel_reps,
                               sleep_cycles)
    n_touch = touched_experts(torch, layers)
    router = router_us(moe, torch, layers, wl, args.kernel_reps, sleep_cycles)
    per_gu, per_dn = expert_bytes(wl)
    avg_touch = sum(n_touch) / len(n_touch)
    gu_bytes, dn_bytes = avg_touch * per_gu, avg_touch * per_dn
    gu_gbps = gu_bytes / (fused_us[0] * 1e3)
    fused_gbps = (gu_bytes + dn_bytes) / ((fused_us[0] + fused_us[1]) * 1e3)
    gemv_gbps = (gu_bytes + dn_bytes) / ((chain_us[2] + chain_us[3]) * 1e3)
    del layers
    torch.cuda.empty_cache()
    return {
        "tokens_per_s": wl.T * args.steps / secs,
        "ms_per_step": 1000.0 * secs / args.steps,
        "roofline": {"kernel": "decode_gate_up_kernel (routing + gate_up + SwiGLU-OAI)",
                     "bound": "hbm", "achieved": round(gu_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gu_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(),
                     "bytes_per_launch": int(gu_bytes), "avg_launch_us": round(fused_us[0], 3)},
        "decode": {"fused": {"gate_up_kernel_us": round(fused_us[0], 3),
                             "down_combine_kernel_us": round(fused_us[1], 3),
                             "weight_GBps": round(fused_gbps, 1),
                             "frac_hbm_peak": round(fused_gbps / HBM_PEAK_GBPS, 4),
                             "per_layer_us": round(1e6 * secs / (args.steps * wl.layers), 3)},
                   "five_call_chain": {"tokens_per_s": round(wl.T * args.steps / secs5, 2),
                                       "per_layer_us": round(1e6 * secs5 / (args.steps * wl.layers), 3),
                                       "route_us": round(chain_us[0], 3),
                                       "bucket_us": round(chain_us[1], 3),
                                       "gemv_gate_up_us": round(chain_us[2], 3),
                                       "gemv_down_us": round(chain_us[3], 3),
                                       "combine_us": round(chain_us[4], 3),
                                       "gemv_weight_GBps": round(gemv_gbps, 1)},
                   "touched_experts_per_layer": avg_touch,
                   "router_us": round(router, 3)},
    }


def bench_t64(moe, synth, torch, args, sleep_cycles):
    """Batched decode T=64 with a hot expert: the five-call chain on the GEMM (tile_m 16) and,
    beside it, the projections on the GEMV engine; weight GB/s over the touched experts."""
    wl = synth.WORKLOADS["decode_t64"]
    log(f"building {wl.layers} layers of {wl.desc}")
    layers = build_layers(moe, synth, torch, wl, "gemm", wl.layers)
    steps = max(10, args.steps // 2)
    secs, _ = graph_time(torch, lambda: [L.chain() for L in layers], steps, args.warmup)
    kt = kernel_times_us(moe, torch, layers, lambda L: L.chain(), 5, args.kernel_reps,
                         sleep_cycles)
    for L in layers:
        L.set_kernel("gemv")
    ktv = kernel_times_us(moe, torch, layers, lambda L: L.gate_up() or L.down(), 2,
                          args.kernel_reps, sleep_cycles)
    n_touch = touched_experts(torch, layers)
    counts = torch.stack([L.csr[0] for L in layers]).cpu()
    router = router_us(moe, torch, layers, wl, args.kernel_reps, sleep_cycles)
    per_gu, per_dn = expert_bytes(wl)
    avg_touch = sum(n_touch) / len(n_touch)
    wbytes = avg_touch * (per_gu + per_dn)
    gbps = wbytes / ((kt[2] + kt[3]) * 1e3)
    gbps_v = wbytes / ((ktv[0] + ktv[1]) * 1e3)
    del layers
    torch.cuda.empty_cache()
    return {
        "workload": wl.desc, "T": wl.T, "layers_rotated": wl.layers,
        "chain": "route, bucket (tile_m 16), mx4_moe_gemm gate_up + SwiGLU-OAI, mx4_moe_gemm "
                 "down, combine; HIP graph",
        "tokens_per_s": round(wl.T * wl.layers * steps / secs, 1),
        "per_layer_chain_us": round(1e6 * secs / (steps * wl.layers), 2),
        "route_us": r1(kt[0], 3), "bucket_us": r1(kt[1], 3), "gate_up_us": r1(kt[2]),
        "down_us": r1(kt[3]), "combine_us": r1(kt[4], 3),
        "touched_experts_per_layer": avg_touch,
        "hot_expert_rows": int(counts[:, wl.hot_expert].float().mean().item()),
        "weight_GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "gemv": {"gate_up_us": r1(ktv[0]), "down_us": r1(ktv[1]),
                 "weight_GBps": round(gbps_v, 1), "frac_hbm_peak": round(gbps_v / HBM_PEAK_GBPS, 4)},
        "router_us": r1(router, 3),
    }


def bench_prefill(moe, synth, torch, args, sleep_cycles, name, with_mx8=True):
    """A prefill workload: the five-call chain on the GEMM (bf16 activations) and the chain
    with MXFP8 activations; expert-GEMM TFLOP/s on live rows, against the bf16 (fp8) peak and
    against the attainable roof min(peak, HBM peak x flops/byte)."""
    wl = synth.WORKLOADS[name]
    log(f"building {wl.layers} layers of {wl.desc}")
    players = build_layers(moe, synth, torch, wl, "gemm", wl.layers)
    p_steps = max(5, args.steps // 5)
    psecs, _ = graph_time(torch, lambda: [L.chain() for L in players], p_steps, args.warmup)
    pkt = kernel_times_us(moe, torch, players, lambda L: L.chain(), 5, args.kernel_reps,
                          sleep_cycles)
    flops = chain_flops(wl)
    n_touch = touched_experts(torch, players)
    per_gu, per_dn = expert_bytes(wl)
    avg_touch = sum(n_touch) / len(n_touch)
    wbytes = avg_touch * (per_gu + per_dn)
    # bytes the layer must move at least: touched weights, x read, h written and read, d
    # written and read, y written, biases
    R = wl.T * wl.k
    act_bytes = (wl.T * wl.dim * 2 + 2 * R * wl.ffn * 2 + 2 * R * wl.dim * 4 + wl.T * wl.dim * 4
                 + avg_touch * (2 * wl.ffn + wl.dim) * 4)
    roof_bf16 = min(BF16_DENSE_TFLOPS, HBM_PEAK_GBPS * 1e-3 * flops / (wbytes + act_bytes))
    t_us = pkt[2] + pkt[3]
    tflops = flops / (t_us * 1e-6) / 1e12
    out = {
        "workload": wl.desc, "T": wl.T, "E": wl.E, "layers_rotated": wl.layers,
        "expert_gemm_TFLOPs": round(tflops, 1),
        "frac_bf16_peak": round(tflops / BF16_DENSE_TFLOPS, 4),
        "attainable_TFLOPs": round(roof_bf16, 1),
        "frac_attainable": round(tflops / roof_bf16, 4),
        "gate_up_us": r1(pkt[2]), "down_us": r1(pkt[3]),
        "route_us": r1(pkt[0], 3), "bucket_us": r1(pkt[1], 3), "combine_us": r1(pkt[4], 3),
        "weight_GBps": round(wbytes / (t_us * 1e3), 1),
        "touched_experts_per_layer": avg_touch,
        "chain_tokens_per_s": round(wl.T * wl.layers * p_steps / psecs, 1),
        "per_layer_chain_us": round(1e6 * psecs / (p_steps * wl.layers), 2),
        "flops_per_layer": flops,
    }
    if with_mx8:
        log(f"{name} with MXFP8 activations (MX-scaled MFMA)")
        for L in players:
            L.alloc_mx8(torch)
        msecs, _ = graph_time(torch, lambda: [L.chain_mx8() for L in players], p_steps,
                              args.warmup)
        mkt = kernel_times_us(moe, torch, players, lambda L: L.chain_mx8(), 6, args.kernel_reps,
                              sleep_cycles)
        mx_tflops = flops / ((mkt[3] + mkt[4]) * 1e-6) / 1e12
        out["mx8"] = {
            "activations": "MXFP8 (E4M3 + e8m0 per 32), v_mfma_scale_f32_16x16x128_f8f6f4",
            "expert_gemm_TFLOPs": round(mx_tflops, 1),
            "frac_fp8_peak": round(mx_tflops / FP8_DENSE_TFLOPS, 4),
            "gate_up_us": r1(mkt[3]), "down_us": r1(mkt[4]), "quantize_x_us": r1(mkt[2]),
            "h_quantized_in": "the gate_up epilogue (MOE_ACT_SWIGLU_OAI_MX8)",
            "chain_tokens_per_s": round(wl.T * wl.layers * p_steps / msecs, 1),
            "per_layer_chain_us": round(1e6 * msecs / (p_steps * wl.layers), 2),
        }
    out["router_us"] = r1(router_us(moe, torch, players, wl, args.kernel_reps, sleep_cycles))
    del players
    torch.cuda.empty_cache()
    return out


def bench_peaks(moe, torch, sleep_cycles):
    """Attained peaks: moe_probe_read over 52.88 MB (a decode layer's touched weights), 423 MB
    (a gpt-oss-20b layer) and 2 GiB, each as 16 buffers read in turn so no read is served by
    the caches; moe_probe_mfma_bf16 on every SIMD."""
    out = {}
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    for label, nbytes in (("52.9MB", 52_876_800), ("423MB", 423_014_400), ("2GiB", 2 << 30)):
        nb = nbytes // 1024 * 1024
        count = 16 if nbytes < (1 << 30) else 2
        bufs = [torch.ones(nb // 4, dtype=torch.int32, device="cuda") for _ in range(count)]
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        best = None
        for wgs in (cus, cus * 4, cus * 8):
            for b in bufs:
                moe.moe_probe_read(b, wgs, sink=sink)
            torch.cuda.synchronize()
            with MARK:
                moe.moe_timing_arm(len(bufs))
                for b in bufs:
                    moe.moe_probe_read(b, wgs, sink=sink)
                ms = moe.moe_timing_read(len(bufs))
                moe.moe_timing_arm(0)
            us = 1000.0 * sum(ms) / len(ms)
            if best is None or us < best[0]:
                best = (us, wgs)
        out[f"read_{label}_GBps"] = round(nb / (best[0] * 1e3), 1)
        del bufs
        torch.cuda.empty_cache()
    wgs, iters = cus * 8, 2000
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    moe.moe_probe_mfma_bf16(wgs, iters, sink=sink)
    torch.cuda.synchronize()
    with MARK:
        moe.moe_timing_arm(4)
        for _ in range(4):
            moe.moe_probe_mfma_bf16(wgs, iters, sink=sink)
        ms = moe.moe_timing_read(4)
        moe.moe_timing_arm(0)
    fl = wgs * 4 * iters * 4 * 32768.0
    out["mfma_bf16_TFLOPs"] = round(fl / (sum(ms) / 4 * 1e-3) / 1e12, 1)
    out["note"] = ("moe_probe_read: grid-stride nontemporal 16-byte loads, best of 1/4/8 "
                   "workgroups per CU; moe_probe_mfma_bf16: v_mfma_f32_32x32x16_bf16 loop, 4 "
                   "independent chains per wavefront, 8 workgroups of 4 wavefronts per CU")
    return out


# ------------------------------------------------------------------------------------------
# CPU oracle baseline
# ------------------------------------------------------------------------------------------

def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _time_decode_layers(oracle, synth, wl, budget_s):
    times = []
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
    return sum(times) / len(times), len(times)


def _time_prefill_sample(oracle, synth, wl, n_experts):
    """The oracle's two projections of a prefill layer on the first n_experts live experts (their
    routed rows), plus route + bucket of the whole layer; returns (seconds of route + bucket,
    seconds of the sample's projections, the sample's routed rows)."""
    tok = synth.tokens(wl, 0)
    W = synth.layer_weights(wl, 0)
    t0 = time.perf_counter()
    ids, w = oracle.route_topk(tok["logits"], wl.k)
    mpad = oracle.mpad_max(wl.T, wl.k, wl.E, wl.tile_m)
    counts, basep, row_tok, pos = oracle.bucket(ids, wl.E, wl.tile_m, mpad)
    t_front = time.perf_counter() - t0
    sub = counts.copy()
    live = [e for e in range(wl.E) if counts[e] > 0][:n_experts]
    sub[[e for e in range(wl.E) if e not in live]] = 0
    t0 = time.perf_counter()
    g, _ = oracle.project(tok["x"], row_tok, W["gate_up"]["q"], W["gate_up"]["s"],
                          W["gate_up"]["bias"], sub, basep, mpad)
    rows = [r for _, r in oracle.live_rows(sub, basep)]
    h = oracle.bf16_round(oracle.swiglu_oai(g[rows], synth.ALPHA, synth.LIMIT))
    import numpy as np
    hh = np.zeros((mpad, wl.ffn), dtype=np.uint16)
    hh[rows] = h
    oracle.project(hh, None, W["down"]["q"], W["down"]["s"], W["down"]["bias"], sub, basep, mpad)
    t_proj = time.perf_counter() - t0
    n_rows = int(sub.sum())
    return t_front, t_proj, n_rows


def cpu_baseline(synth, budget_s):
    """The CPU oracle (as it stands) on bounded samples: the decode workload on one host thread
    and on all of them (numpy's BLAS threads), the pp512 and 120b prefill layers on all."""
    import oracle
    from threadpoolctl import threadpool_limits
    wl = synth.WORKLOADS["decode_t1"]
    cores = host_cores()
    with threadpool_limits(limits=1):
        t1, n1 = _time_decode_layers(oracle, synth, wl, budget_s)
    with threadpool_limits(limits=cores):
        ta, na = _time_decode_layers(oracle, synth, wl, budget_s)
    prefill = {}
    for name in ("prefill_pp512", "prefill_120b_t2048"):   # all host threads only
        pw = synth.WORKLOADS[name]
        with threadpool_limits(limits=cores):
            tf, tp, n_rows = _time_prefill_sample(oracle, synth, pw, 4)
        R = pw.T * pw.k
        layer_s = tf + tp * R / n_rows               # the projections scale with the routed rows
        gflops = chain_flops(pw) * n_rows / R / tp / 1e9
        prefill[name] = {"tokens_per_s": round(pw.T / layer_s, 2),
                         "s_per_layer": round(layer_s, 2), "GFLOPs": round(gflops, 2),
                         "cores": cores,
                         "sample": f"route + bucket of layer 0 ({tf:.2f} s) and the two "
                                   f"projections of its first 4 live experts ({n_rows} routed "
                                   f"rows, {tp:.2f} s), scaled to the layer's {R} rows"}
    return {"value": round(wl.T / (ta * wl.layers), 4), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"oracle.chain (float64 numpy, {cores} threads) on 1 token through layers "
                      f"0..{na - 1} of the 24-layer decode workload; {ta * 1e3:.0f} ms per layer, "
                      f"scaled to 24 layers",
            "single_thread": {"value": round(wl.T / (t1 * wl.layers), 4), "unit": "tokens/s",
                              "cores": 1, "ms_per_layer": round(t1 * 1e3, 1),
                              "sample": f"layers 0..{n1 - 1}"},
            **prefill, "nproc": os.cpu_count(), "cpu_model": cpu_model()}


# ------------------------------------------------------------------------------------------
# counter passes (rocprofv3 --pmc)
# ------------------------------------------------------------------------------------------

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


def copy_kernel_pass(torch):
    """A plain copy of known size (reads 64 MiB, writes 64 MiB) three times: the counters' scale."""
    src = torch.ones(16 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()


def counter_pass(moe, synth, torch, name, with_mx8=False):
    """Workload of the rocprofv3 --pmc passes: the copy kernel, then the workload's chain over
    its layers twice (decode_t1: mx4_moe_decode over 8 layers; the others: the five-call chain,
    and with_mx8 the MXFP8 chain as well)."""
    copy_kernel_pass(torch)
    wl = synth.WORKLOADS[name]
    if name == "decode_t1":
        layers = build_layers(moe, synth, torch, wl, "gemv", 8)
        for _ in range(2):
            for L in layers:
                L.decode()
    else:
        layers = build_layers(moe, synth, torch, wl, "gemm", wl.layers)
        for _ in range(2):
            for L in layers:
                L.chain()
        torch.cuda.synchronize()
        if with_mx8:
            for L in layers:
                L.alloc_mx8(torch)
            for _ in range(2):
                for L in layers:
                    L.chain_mx8()
    torch.cuda.synchronize()
    log(f"counter pass {name} done")


def trace_summary(path):
    """Per-kernel duration statistics of a rocprofv3 kernel trace (CSV), over the dispatches
    inside the marked timing regions (between consecutive one-workgroup probe_read_kernel
    dispatches) and over all dispatches. Returns {kernel: {...}}."""
    import csv
    import statistics
    rows = list(csv.DictReader(open(path)))

    def grid(r):
        for key in ("Grid_Size_X", "Grid_Size"):
            if key in r and r[key]:
                return int(r[key])
        return -1

    def wg(r):
        for key in ("Workgroup_Size_X", "Workgroup_Size"):
            if key in r and r[key]:
                return int(r[key])
        return -2

    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    inside, marked, allk = False, {}, {}
    for r in rows:
        name = r["Kernel_Name"]
        if "probe_read_kernel" in name and grid(r) == wg(r):
            inside = not inside
            continue
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        allk.setdefault(name, []).append(dur)
        if inside:
            marked.setdefault(name, []).append(dur)
    out = {}
    for name, ds in marked.items():
        a = allk[name]
        out[name] = {"marked_calls": len(ds), "marked_mean_us": statistics.fmean(ds),
                     "marked_median_us": statistics.median(ds), "marked_min_us": min(ds),
                     "marked_max_us": max(ds), "all_calls": len(a),
                     "all_mean_us": statistics.fmean(a)}
    return out


def main():
    global ROCTX, MARK
    if len(sys.argv) == 3 and sys.argv[1] == "--trace-summary":
        for name, st in sorted(trace_summary(sys.argv[2]).items(),
                               key=lambda kv: -kv[1]["marked_mean_us"] * kv[1]["marked_calls"]):
            print(json.dumps({"kernel": name, **{k: round(v, 3) for k, v in st.items()}}))
        return
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
    ROCTX = Roctx()
    MARK = Marked(moe, torch)
    if args.counter_pass_prefill:
        counter_pass(moe, synth, torch, "prefill_pp512", with_mx8=True)
        return
    if args.counter_pass:
        counter_pass(moe, synth, torch, args.counter_pass)
        return
    sleep_cycles = sleep_cycles_for(torch, 20.0)
    wl = synth.WORKLOADS["decode_t1"]
    result = {
        "metric": "MoE chain tokens/s; decode mx4 weight GB/s; pp512 expert GEMM TFLOP/s (1 GPU)",
        "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gpt-oss-20b-shaped decode, T=1, 24 distinct MoE layers per step",
                   "E": wl.E, "dim": wl.dim, "ffn": wl.ffn, "k": wl.k, "T": wl.T,
                   "layers": wl.layers, "weights": "mxfp4", "accumulate": "f32",
                   "chain": "mx4_moe_decode (2 launches per layer)", "graph": "hip graph replay"},
    }
    if "decode" in args.parts:
        d = bench_decode(moe, synth, torch, args, sleep_cycles)
        result["value"] = round(d["tokens_per_s"], 2)
        result["ms_per_step"] = round(d["ms_per_step"], 4)
        result["roofline"] = d["roofline"]
        result["decode"] = d["decode"]
    if "t64" in args.parts:
        result["decode_t64"] = bench_t64(moe, synth, torch, args, sleep_cycles)
    if "pp512" in args.parts:
        result["prefill_pp512"] = bench_prefill(moe, synth, torch, args, sleep_cycles,
                                                "prefill_pp512")
    if "120b" in args.parts:
        result["prefill_120b_t2048"] = bench_prefill(moe, synth, torch, args, sleep_cycles,
                                                     "prefill_120b_t2048")
    if "peaks" in args.parts:
        log("attained peaks")
        result["attained_peaks"] = bench_peaks(moe, torch, sleep_cycles)
    if "cpu" in args.parts:
        log("timing the CPU oracle on bounded samples")
        result["cpu_baseline"] = cpu_baseline(synth, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
