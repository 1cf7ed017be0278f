// mx4_moe_decode_persistent: the routed MXFP4 expert chain of a few tokens in ONE launch, with
// every weight byte of the layer in flight as soon as the routing is known.
//
// Sources: PR #3579 "dasLLAMA gpt-oss arc", PR body section "Fused MoE expert chain" and the
// fused chain commit (stage 1: gate and up rows + bias + activation; stage 2: every routed
// expert's down row + bias and the routing-weighted sum in slot order), Metal fusion-lane commit
// (bias-seeded accumulators); PR #3558 section "gpt-oss: mx4 kernels to the lab-winning shape"
// (the routed-expert GEMV: every weight byte loaded once).
//
// At decode sizes a layer is a ~53 MB weight stream (gpt-oss-20b shape, one token: 4 experts x
// 13.2 MB), which one plain read kernel streams in ~9 us; what a launch per stage adds is the
// round trip before each stream (routing before gate_up, the expert ids and h before down) and
// the drain at each launch boundary. Here one resident grid (one workgroup per CU) does it all:
//  * A gate_up unit is 16 weight rows (8 gate rows and the 8 up rows of the same h columns) of
//    one pick over the whole reduction, streamed by one wavefront through a ring of 12 chunks
//    in registers (refilled in place as each group of 4 chunks is consumed), so a wavefront
//    keeps 12 KB in flight and computes as its bytes arrive, then applies the clamped
//    SwiGLU-OAI itself and stores h with device-scope stores.
//  * A down tile is 16 output rows of one token over every slot: 2k wavefronts, each holding
//    one slot's rows over half the reduction (12 chunks) in registers from the start. The tile
//    stays in one workgroup, so d and the slot-order combine stay on chip.
//  * Workgroup b owns down tiles b, b + G, ... and a contiguous range of gate_up units in
//    proportion to its wavefronts not holding a down tile.
//  * Every wavefront routes the token of its own first unit itself (the pick order of
//    moe_route_topk), then issues that unit's loads: no barrier before the weight stream, as
//    the wavefronts of a workgroup start at different times.
//  * When a workgroup's h rows are stored it counts itself in the caller's workspace (two
//    levels, so no word takes more than ~32 atomics); the down wavefronts wait (one thread
//    polls, bounded) until every workgroup has counted, stage h with device-coherent loads and
//    multiply their registers' weights by it.
//  * No workgroup waits for anything but that count, which every workgroup reaches before it
//    waits, and the host sizes the grid to what can be resident at once; the wait is bounded all
//    the same (an error flag in the workspace instead of a hang).
#include <mutex>

#include "gemv_core.hpp"
#include "launch.hpp"
#include "route_core.hpp"

namespace moe {

constexpr int kLyWaves = 12;                 // 3 per SIMD (168 registers each)
constexpr int kLyThreads = 64 * kLyWaves;
constexpr int kLyMaxC = 24;                  // chunks of the reduction (K <= 3072)
constexpr int kLyRing = 12;                  // ring slots (3 groups of 4 chunks)
// Workspace words (u32; zero before the first call, then the library's own state). The "h is
// complete" signal is counted in two levels, so that no word takes more than ~32 atomic adds
// and ~32 pollers: workgroup b adds 1 to the counter of its group b % 8 (the XCD the hardware
// deals it to); the last of a group adds 1 to kLyDone (and re-zeroes its group's counter);
// the last group re-zeroes kLyDone, advances the epoch and publishes it in each group's go
// word, which that group's down workgroups poll. Epochs are never re-zeroed, so no word has to
// be reset after the pollers have seen it.
constexpr int kLyDone = 0, kLyEpoch = 1, kLyErr = 3;
constexpr int kLyGroups = 8;
constexpr int kLyLine = 32;                  // words between counters (128-byte lines)
constexpr int kLyCnt = kLyLine;              // group counters: kLyCnt + kLyLine * g
constexpr int kLyGo = kLyLine * (1 + kLyGroups);   // group go words: kLyGo + kLyLine * g
static_assert(kLyGo + kLyLine * kLyGroups <= MOE_DECODE_WS_WORDS, "workspace size");
constexpr uint32_t kLySpinMax = 1u << 21;    // polls of ~0.3 us each, about a second

// First gate_up unit of workgroup b. Workgroup j holds a down tile (2k wavefronts) from the
// start if j < V, and its other wavefronts take gate_up units: the units are dealt in
// contiguous ranges in proportion to those free wavefronts, so that at gpt-oss decode shape
// every unit has a wavefront of its own from the start (no second round at the end of the
// stream). start(G) = U; non-decreasing in b.
__host__ __device__ inline int64_t ly_unit_start(int64_t b, int64_t G, int64_t U, int64_t V,
                                                 int64_t wd) {
  const int64_t cap_b = b * kLyWaves - wd * (b < V ? b : V);
  const int64_t cap_g = G * kLyWaves - wd * (G < V ? G : V);
  return U * cap_b / cap_g;
}

// One chunk (16 rows x 128 k) of a wavefront's weights times the activation row at xl (LDS,
// the chunk's first block for this lane's k-group): 4 MFMA k-steps, two accumulator chains.
// Every lane reads the activation row: only output column 0 is used, and column c of the
// product depends only on B column c, so the other columns may hold the same values; the 16
// lanes of a k-group read one address, which LDS broadcasts.
__device__ __forceinline__ void ly_chunk(const u32x4_t& wq, float scl, const uint8_t* xl,
                                         f32x4_t& acc0, f32x4_t& acc1) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4_t& acc = (t & 1) ? acc1 : acc0;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        dequant8(wq[t], scl), *reinterpret_cast<const bf16x8_t*>(xl + 16 * t), acc, 0, 0, 0);
  }
}

// One wavefront's weights: 16 rows of one expert over chunks [cbase, cend) of the reduction
// (cbase a multiple of 4), in a ring of 12 chunk slots. Group g (chunks cbase + 4g..: one scale
// dwordx4, then 4 nibble loads) goes to slots 4(g % 3)... A gate_up unit streams all of K
// (cbase 0, up to 24 chunks): group g + 3 is issued into group g's slots as soon as group g is
// consumed, so the wavefront keeps 12 KB in flight and computes as its bytes arrive. A down
// item holds its half of K (12 chunks, groups 0-2) from the start until h is ready. Every group
// issues its 5 loads (past cend they read zeros through out-of-range offsets), so the number of
// loads issued after a group is known and each step waits for exactly its own group.
// Straight-line (compile-time groups): no loop header for the compiler to be conservative at.
// Both roles use this one register set (the compiler cannot tell that a wavefront takes only
// one of them).
struct LyRing {
  __amdgpu_buffer_rsrc_t rq, rs;
  uint32_t wo, wol, so;
  int C, N, cbase, cend;
  u32x4_t wq[kLyRing];
  uint32_t sc[kLyRing];

  __device__ __forceinline__ void init(const uint8_t* __restrict__ q,
                                       const uint8_t* __restrict__ s, int e, int n, bool valid,
                                       int N_, int K, int cb, int ce) {
    e = __builtin_amdgcn_readfirstlane(e);
    N_ = __builtin_amdgcn_readfirstlane(N_);
    K = __builtin_amdgcn_readfirstlane(K);
    cbase = __builtin_amdgcn_readfirstlane(cb);
    cend = __builtin_amdgcn_readfirstlane(ce);
    const int lg = (int)(threadIdx.x & 63) >> 4;
    N = N_;
    const int KB = K >> 5;
    C = (KB + kChunkBlocks - 1) / kChunkBlocks;
    const int G = scale_row_bytes(KB) / 16;
    const int wlast = KB - (C - 1) * kChunkBlocks;
    rq = make_rsrc(q + 16 * (size_t)e * N * KB, (uint32_t)N * KB * 16);
    rs = make_rsrc(s + (size_t)e * N * G * 16, (uint32_t)N * G * 16);
    wo = valid ? ((uint32_t)n * kChunkBlocks + lg) * 16 : kOOB;
    wol = (valid && lg < wlast) ? ((uint32_t)n * wlast + lg) * 16 : kOOB;
    so = valid ? (uint32_t)n * 16 : kOOB;
  }

  template <int g>
  __device__ __forceinline__ void load_group() {
    constexpr int base = 4 * (g % 3);
    const int c0 = cbase + 4 * g;
    const u32x4_t v = buf_load16_nt(rs, c0 < cend ? so : kOOB, (uint32_t)(c0 >> 2) * N * 16);
    sc[base + 0] = v[0];
    sc[base + 1] = v[1];
    sc[base + 2] = v[2];
    sc[base + 3] = v[3];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = c0 + kk;
      const uint32_t off = (c >= cend) ? kOOB : (c < C - 1 ? wo : wol);
      wq[base + kk] = buf_load16_nt(rq, off, (uint32_t)c * N * (kChunkBlocks * 16));
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  __device__ __forceinline__ void start() {
    load_group<0>();
    load_group<1>();
    load_group<2>();
  }

  // group g: wait until it has landed (LATER loads were issued after it), compute its chunks
  // against the activation row xrow (LDS), then (REFILL) issue group g + 3 into its slots
  template <int g, int LATER, bool REFILL>
  __device__ __forceinline__ void step(const uint8_t* xrow, f32x4_t& acc0, f32x4_t& acc1) {
    constexpr int base = 4 * (g % 3);
    const int lg = (int)(threadIdx.x & 63) >> 4;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(LATER));
    __builtin_amdgcn_sched_barrier(0);
    if (cbase + 4 * g < cend) {   // uniform
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int c = cbase + 4 * g + kk;
        // past cend: zero weights and a zero scale operand; the row reads stay inside the
        // zero-padded staging area
        const uint32_t eb = c < cend ? __builtin_amdgcn_ubfe(sc[base + kk], 8 * lg, 8) : 0u;
        ly_chunk(wq[base + kk], e8m0_scale_operand(eb),
                 xrow + ((size_t)c * kChunkBlocks + lg) * 64, acc0, acc1);
        __builtin_amdgcn_sched_barrier(0);   // one chunk's reads and converts live at a time
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (REFILL) load_group<g + 3>();
  }

  // a gate_up unit: all six groups through the ring (acc0 seeded with the bias by the caller)
  __device__ __forceinline__ void run_all(const uint8_t* xrow, f32x4_t& acc0, f32x4_t& acc1) {
    static_assert(kLyMaxC == 24, "six groups");
    step<0, 10, true>(xrow, acc0, acc1);
    step<1, 10, true>(xrow, acc0, acc1);
    step<2, 10, true>(xrow, acc0, acc1);
    step<3, 10, false>(xrow, acc0, acc1);
    step<4, 5, false>(xrow, acc0, acc1);
    step<5, 0, false>(xrow, acc0, acc1);
  }

  // a down item: the three groups it holds
  __device__ __forceinline__ void run_held(const uint8_t* xrow, f32x4_t& acc0, f32x4_t& acc1) {
    step<0, 10, false>(xrow, acc0, acc1);
    step<1, 5, false>(xrow, acc0, acc1);
    step<2, 0, false>(xrow, acc0, acc1);
  }
};

struct LyArgs {
  const float* logits;
  const uint16_t* x;
  const uint8_t *gq, *gs, *dq, *ds;
  const float *gb, *db;
  int T, E, k, D, F, N;
  float alpha, limit;
  int U1, Ut, U, TD, V, xrows;
  int32_t *ids, *counts, *basep, *row_tok, *pos;
  float* w;
  uint16_t* h;
  float *d, *y;
  uint32_t* ws;
};

// LDS layout (bytes), shared by host and device
struct LyLds {
  int rowb, hrow, areg, roff, koff, pkoff, pvoff, total;
  __host__ __device__ LyLds(int D, int F, int k, int T, int xrows) {
    // activation rows in 1 KB DMA pieces, each row zero-padded to whole pieces: a group of 4
    // chunks (16 blocks, 1 KB of bf16) never reads past its row's pieces, so reads past the
    // row's end (blocks past K, chunks past the range) see zeros
    rowb = ((D * 2) + 1023) & ~1023;                       // x rows (gate_up phase)
    hrow = ((F * 2) + 1023) & ~1023;                       // h rows, one per slot (down phase)
    areg = xrows * rowb > k * hrow ? xrows * rowb : k * hrow;
    roff = areg;                                           // down partial rows: 1 KB per wave
    koff = roff + kLyWaves * 1024;                         // rank keys: 512 B per wave
    pkoff = koff + kLyWaves * 512;                         // picks [T][k]
    pvoff = pkoff + T * k * 4;                             // picked logits [T][k]
    total = pvoff + T * k * 4;
  }
};

__global__ void __launch_bounds__(kLyThreads)
decode_layer_kernel(LyArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const LyLds L(a.D, a.F, a.k, a.T, a.xrows);
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  const int tid = (int)threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int k = a.k, F = a.F, D = a.D;
  int* const picks = reinterpret_cast<int*>(lds + L.pkoff);
  float* const pval = reinterpret_cast<float*>(lds + L.pvoff);   // the picked logits
  const int C1 = (D / 32 + kChunkBlocks - 1) / kChunkBlocks;
  const int C2 = (F / 32 + kChunkBlocks - 1) / kChunkBlocks;

  // this workgroup's work
  const int u0 = (int)ly_unit_start(b, G, a.U, a.V, 2 * k);
  const int u1 = (int)ly_unit_start(b + 1, G, a.U, a.V, 2 * k);
  const int nd = b < a.V ? (a.V - 1 - b) / G + 1 : 0;      // down tiles b, b + G, ...
  const int wd = nd > 0 ? 2 * k : 0;                        // waves holding a down item
  const int wg = kLyWaves - wd;                             // gate_up waves
  const int tf = u0 < u1 ? u0 / a.Ut : 0;                   // x rows: tokens tf..

  // 1. the x rows of the range's tokens (no routing needed); past each row, up to its 1 KB
  // piece, the copy writes zeros
  if (u0 < u1) {
    const int tl = (u1 - 1) / a.Ut;
    const int pieces = L.rowb >> 10;
    for (int t = tf; t <= tl; ++t) {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(a.x + (size_t)t * D, (uint32_t)D * 2);
      for (int i = wave; i < pieces; i += kLyWaves)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(lds + (t - tf) * L.rowb + i * 1024), 16,
            (uint32_t)i * 1024 + (uint32_t)lane * 16, 0, 0, 0);
    }
  }

  // 2. routing, by every wavefront for itself: the expert of its own first unit, and for
  // wavefront w the picks of tokens w, w + 12, ..., published in LDS for the later units, the
  // combine and the caller's copy. All of it before the unit's weight loads, which complete
  // after it. The logits rows (E <= 64) come by LDS-DMA into the wavefront's own 1 KB (of the
  // down partials area, unused until then; zeros past E), all in flight at once, and are ranked
  // from there: one memory round trip.
  const int gw = wave - wd;                 // gate_up wavefront index (if >= 0)
  int first_t = -1, first_s = 0;            // token and slot of this wavefront's first unit
  if (wave < wd) {
    first_t = b / a.TD;
    first_s = wave >> 1;
  } else if (u0 + gw < u1) {
    const int u = u0 + gw;
    first_t = u / a.Ut;
    first_s = (u - first_t * a.Ut) / a.U1;
  }
  float* const lrows = reinterpret_cast<float*>(lds + L.roff + wave * 1024);   // 4 rows of 64
  {
    auto dma_row = [&](int t, int j) {
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.logits + (size_t)t * a.E, (uint32_t)a.E * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rl, (__attribute__((address_space(3))) void*)(lrows + 64 * j), 4, (uint32_t)lane * 4, 0,
          0, 0);
    };
    if (first_t >= 0) dma_row(first_t, 0);
    for (int t = wave, j = 1; t < a.T; t += kLyWaves, ++j) dma_row(t, j);   // j <= 2 (T <= 16)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
  // lanes < k: pick `lane` of the token staged in row j
  uint64_t* const keys = reinterpret_cast<uint64_t*>(lds + L.koff + wave * 512);
  auto route = [&](int j, int& my_id, float& my_v) {
    const float* row = lrows + 64 * j;
    const int rank = wave_rank_lds(row, keys, a.E);
    my_id = 0;
    for (int r = 0; r < k; ++r) {
      const int id = rank_pick(rank, r);
      if (lane == r) my_id = id;
    }
    my_v = row[min(max(my_id, 0), kWave - 1)];
  };
  int first_e = 0;
  bool have_first = false;
  for (int t = wave, j = 1; t < a.T; t += kLyWaves, ++j) {   // publish the picks of its tokens
    int id;
    float v;
    route(j, id, v);
    if (lane < k) {
      picks[t * k + lane] = min(max(id, 0), a.E - 1);   // in [0, E) by the total order
      pval[t * k + lane] = v;
    }
    if (t == first_t) {
      first_e = __shfl(id, first_s);
      have_first = true;
    }
  }
  if (first_t >= 0 && !have_first) {
    int id;
    float v;
    route(0, id, v);
    first_e = __shfl(id, first_s);
  }
  first_e = min(max(first_e, 0), a.E - 1);

  // 3. every wavefront issues the loads of its first unit; its bias seeds come through the
  // scalar cache, outside the in-order count of the weight loads
  LyRing un;   // this wavefront's weights (a gate_up unit or a down item)
  f32x4_t seed = {0.0f, 0.0f, 0.0f, 0.0f};
  auto gate_up_seed = [&](int u, int e) {   // through the scalar cache (scalar_seed16)
    const int t = u / a.Ut;
    const int j = __builtin_amdgcn_readfirstlane(((u - t * a.Ut) % a.U1) * 8);
    f32x4_t sd = {0.0f, 0.0f, 0.0f, 0.0f};
    if (a.gb) {   // j + 8 <= F: F % 8 == 0
      const float* br = a.gb + (size_t)__builtin_amdgcn_readfirstlane(e) * a.N + j;
      float b4[4];
      scalar_seed16(br, br + F, b4);
      sd = f32x4_t{b4[0], b4[1], b4[2], b4[3]};
    }
    return sd;
  };
  auto gate_up_start = [&](int u, int e) {
    const int t = u / a.Ut;
    const int j = (u - t * a.Ut) % a.U1;
    const int jj = j * 8 + (lr & 7);
    un.init(a.gq, a.gs, e, lr < 8 ? jj : F + jj, true, a.N, D, 0, C1);
    un.start();
  };
  auto down_seed = [&](int tile, int e) {   // the bias seeds half 0's sums; D % 16 == 0
    f32x4_t sd = {0.0f, 0.0f, 0.0f, 0.0f};
    if ((wave & 1) == 0 && a.db) {
      const float* br =
          a.db + (size_t)__builtin_amdgcn_readfirstlane(e) * D + __builtin_amdgcn_readfirstlane(tile) * 16;
      float b4[4];
      scalar_seed16(br, br + 8, b4);
      sd = f32x4_t{b4[0], b4[1], b4[2], b4[3]};
    }
    return sd;
  };
  auto down_start = [&](int tile, int e) {
    const int n = tile * 16 + lr;
    int cb, ce, Cp;
    k_part_range(C2, wave & 1, 2, cb, ce, Cp);
    un.init(a.dq, a.ds, e, n, n < D, D, F, cb, ce);
    un.start();
  };
  if (wave < wd) {
    seed = down_seed(b - first_t * a.TD, first_e);
    down_start(b - first_t * a.TD, first_e);
  } else if (first_t >= 0) {
    seed = gate_up_seed(u0 + gw, first_e);
    gate_up_start(u0 + gw, first_e);
  }
  // the x rows (issued before the routing and the unit loads) have landed; picks published
  if (first_t >= 0)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(15));   // all but the unit's 15 loads
  else
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // 4. gate_up units u0 + gw, u0 + gw + wg, ...: stream, SwiGLU-OAI, store h
  if (wave >= wd) {
    for (int u = u0 + gw; u < u1; u += wg) {
      if (u != u0 + gw) {   // a later unit (more units than wavefronts): its loads now
        const int t = u / a.Ut;
        const int e = picks[t * k + (u - t * a.Ut) / a.U1];
        seed = gate_up_seed(u, e);
        gate_up_start(u, e);
      }
      const int t = u / a.Ut;
      const int r = u - t * a.Ut;
      const int slot = r / a.U1, j = r - slot * a.U1;
      f32x4_t acc0 = seed, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
      un.run_all(lds + (t - tf) * L.rowb, acc0, acc1);
      acc0 += acc1;
      // SwiGLU-OAI: lanes 0 and 16 hold gate rows 0-3 / 4-7, lanes 32 and 48 the up rows
      float up[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) up[i] = __shfl_xor(acc0[i], 32);
      if (lr == 0 && lg < 2) {
        const int j0 = j * 8 + 4 * lg;
        uint32_t hb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          hb[i] = f32_to_bf16_bits(swiglu_oai(acc0[i], up[i], a.alpha, a.limit));
        uint32_t* d32 = reinterpret_cast<uint32_t*>(a.h + ((size_t)t * k + slot) * F + j0);
        __hip_atomic_store(d32, hb[0] | (hb[1] << 16), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(d32 + 1, hb[2] | (hb[3] << 16), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  // 5. this workgroup's h rows are stored (acknowledged) -> count it. The down waves' weight
  // loads are still in flight and are not waited for here.
  if (wave >= wd) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  // the poller's call epoch, read before this workgroup counts (so before the count can
  // complete and the epoch advance); the down wavefronts are idle here
  uint32_t epoch = 0;
  if (nd > 0 && tid == 0)
    epoch = __hip_atomic_load(a.ws + kLyEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_barrier();
  const int grp = b % kLyGroups;
  if (tid == 64 * wd) {   // a gate_up wavefront's lane 0 (wd <= 12 < kLyWaves)
    const int ngroups = G < kLyGroups ? G : kLyGroups;
    const uint32_t in_grp = (uint32_t)((G - 1 - grp) / kLyGroups + 1);
    if (__hip_atomic_fetch_add(a.ws + kLyCnt + kLyLine * grp, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) == in_grp - 1) {
      __hip_atomic_store(a.ws + kLyCnt + kLyLine * grp, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (__hip_atomic_fetch_add(a.ws + kLyDone, 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)ngroups - 1) {
        __hip_atomic_store(a.ws + kLyDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t next_epoch =
            __hip_atomic_fetch_add(a.ws + kLyEpoch, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT) + 1u;
        for (int g2 = 0; g2 < ngroups; ++g2)
          __hip_atomic_store(a.ws + kLyGo + kLyLine * g2, next_epoch, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  // 6. down tiles: wait once for every workgroup's h, then each tile
  if (nd > 0) {
    if (tid == 0) {
      uint32_t it = 0;
      while (__hip_atomic_load(a.ws + kLyGo + kLyLine * grp, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) != epoch + 1) {
        __builtin_amdgcn_s_sleep(4);
        if (++it == kLySpinMax) {
          __hip_atomic_store(a.ws + kLyErr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    int t_staged = -1;
    f32x4_t* const red = reinterpret_cast<f32x4_t*>(lds + L.roff);
    for (int q = 0; q < nd; ++q) {
      const int v = b + q * G;
      const int t = v / a.TD, tile = v - t * a.TD;
      int cb, ce, Cp;
      k_part_range(C2, wave & 1, 2, cb, ce, Cp);
      if (q > 0 && wave < wd) {   // later tiles: their rows now (the first one is in flight)
        const int e = picks[t * k + (wave >> 1)];
        seed = down_seed(tile, e);
        down_start(tile, e);
      }
      if (t != t_staged) {
        // the token's k rows of h (written by other workgroups of this launch) into LDS
        __syncthreads();   // (q == 0: the poll is done; else: the previous tile's reads are)
        // LDS-DMA loads with the device-coherent bit (sc1, as the device-scope stores that wrote
        // h), all in flight at once; each slot's row zero-padded past its F values
        const int per_row = L.hrow >> 10;
        for (int i = wave; i < k * per_row; i += kLyWaves) {
          const int sl = i / per_row, pc = i - sl * per_row;
          const __amdgpu_buffer_rsrc_t rh =
              make_rsrc(a.h + ((size_t)t * k + sl) * F, (uint32_t)F * 2);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rh, (__attribute__((address_space(3))) void*)(lds + i * 1024), 16,
              (uint32_t)pc * 1024 + (uint32_t)lane * 16, 0, 0, 16);
        }
        t_staged = t;
      }
      __syncthreads();
      if (wave < wd) {
        const int sl = wave >> 1;
        f32x4_t acc0 = seed, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
        un.run_held(lds + (size_t)sl * L.hrow, acc0, acc1);   // ce - cb <= 12 chunks
        red[wave * 64 + lane] = acc0 + acc1;
      }
      __syncthreads();
      if (wave == 0) {   // d of each slot (halves in order), y = slot-order sum of w * d
        const float wt = topk_weight(lane < k ? pval[t * k + lane] : 0.0f, k);
        float yv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int sl = 0; sl < k; ++sl) {
          const f32x4_t ds = red[(2 * sl) * 64 + lane] + red[(2 * sl + 1) * 64 + lane];
          const float wsl = __shfl(wt, sl);
#pragma unroll
          for (int i = 0; i < 4; ++i) yv[i] = fmaf(wsl, ds[i], yv[i]);
          if (a.d && lr == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int nn = tile * 16 + 4 * lg + i;
              if (nn < D) a.d[((size_t)t * k + sl) * D + nn] = ds[i];
            }
          }
        }
        if (lr == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int nn = tile * 16 + 4 * lg + i;
            if (nn < D) a.y[(size_t)t * D + nn] = yv[i];
          }
        }
      }
    }
  }

  // 7. the routing and the CSR with tile 1 for the caller, from the picks (last workgroup)
  if (b == G - 1) {
    __syncthreads();
    const int R = a.T * k;
    for (int t = wave; t < a.T; t += kLyWaves) {
      const float wt = topk_weight(lane < k ? pval[t * k + lane] : 0.0f, k);
      if (lane < k) {
        a.ids[t * k + lane] = picks[t * k + lane];
        a.w[t * k + lane] = wt;
      }
    }
    for (int e = tid; e < a.E; e += kLyThreads) {
      int c = 0, before = 0;
      for (int r = 0; r < R; ++r) {
        c += picks[r] == e;
        before += picks[r] < e;   // a token picks an expert at most once
      }
      a.counts[e] = c;
      a.basep[e] = before;
      if (e == a.E - 1) a.basep[a.E] = R;
    }
    for (int r = tid; r < R; r += kLyThreads) {
      // CSR row of (t, s): after every routed row of a lower expert and every earlier token
      // routed to the same expert
      const int e = picks[r], t = r / k;
      int p = 0;
      for (int r2 = 0; r2 < R; ++r2) p += (picks[r2] < e) | ((picks[r2] == e) & (r2 / k < t));
      a.pos[r] = p;
      a.row_tok[p] = t;
    }
  }
}

}  // namespace moe

// Launch plan of mx4_moe_decode_persistent (host): 0 if the one-launch kernel applies, with
// its grid, LDS and work sizes in *a / *G / *lds; else the caller runs the two launches.
namespace moe {
int layer_plan(int64_t T, int E, int k, int D, int F, int max_workgroups, LyArgs* a, int* G,
               size_t* lds) {
  a->U1 = (F + 7) / 8;
  a->Ut = k * a->U1;
  a->U = (int)T * a->Ut;
  a->TD = (D + 15) / 16;
  a->V = (int)T * a->TD;
  // 2k down waves per tile and at least 4 gate_up waves; h stored 4 columns at a time; a whole
  // gate_up reduction in the ring and half of a down reduction in one wavefront
  // (and E <= 64: a logits row ranked by one wavefront from LDS)
  if (2 * k > kLyWaves - 4 || (F & 7) || D > 32 * 4 * kLyMaxC || F > 32 * 4 * kLyMaxC ||
      E > kWave)
    return 1;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  int64_t g = cus;   // one workgroup per CU
  if (max_workgroups > 0 && g > max_workgroups) g = max_workgroups;
  // the most tokens one workgroup's range spans (its x rows are staged together)
  int xrows = 1;
  for (int64_t b = 0; b < g; ++b) {
    const int64_t u0 = ly_unit_start(b, g, a->U, a->V, 2 * k);
    const int64_t u1 = ly_unit_start(b + 1, g, a->U, a->V, 2 * k);
    if (u1 > u0 && (u1 - 1) / a->Ut - u0 / a->Ut + 1 > xrows)
      xrows = (int)((u1 - 1) / a->Ut - u0 / a->Ut + 1);
  }
  a->xrows = xrows;
  const LyLds L(D, F, k, (int)T, xrows);
  *lds = (size_t)L.total;
  if (L.total > 64 * 1024) return 1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&decode_layer_kernel), kLyThreads, *lds) !=
          hipSuccess)
    return -1;
  if (per_cu < 1) return 1;
  *G = (int)g;
  return 0;
}
}  // namespace moe

int moe_launch_decode_two(const float* logits, const uint16_t* x, int64_t T, int E, int k,
                          const mx4_experts* w_gu, const mx4_experts* w_dn, float alpha,
                          float limit, int32_t* ids, float* w, int32_t* counts, int32_t* basep,
                          int32_t* row_tok, int32_t* pos, uint16_t* h, float* d, float* y,
                          hipStream_t stream);

namespace {

// Library-held workspace of mx4_moe_decode_persistent_static. A file-scope device array exists
// once on every GPU the library runs on, each copy at its own device address; host code uses
// only that address (from hipGetSymbolAddress, once per device), never the array's name.
static __device__ __align__(256) uint32_t scratch[MOE_DECODE_WS_WORDS];
static_assert(moe::kLyGo + moe::kLyLine * moe::kLyGroups <= MOE_DECODE_WS_WORDS,
              "the layer kernel's counters fit the workspace");

std::mutex g_scratch_mu;
uint32_t* g_scratch[moe::kMaxDevices];   // device address of `scratch`, per device

// This device's copy of `scratch` (looked up on the first call on the device), or NULL.
uint32_t* scratch_ptr() {
  const int slot = moe::device_slot();
  if (slot < 0) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[slot]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[slot] = static_cast<uint32_t*>(p);
  }
  return g_scratch[slot];
}

// Zero fill of n words (a kernel, not a memset node: callers may capture the call in a graph).
__global__ void __launch_bounds__(256) fill_zero_u32(uint32_t* __restrict__ p, int n) {
  for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += (int)(gridDim.x * blockDim.x))
    p[i] = 0u;
}

// Shared body of both entry points. ws: the caller's workspace, or NULL for the library's own
// (zeroed before the layer kernel on every call that launches it).
int decode_persistent(const float* logits, const uint16_t* x, int64_t T, int E, int k,
                      const mx4_experts* w_gu, const mx4_experts* w_dn, float alpha, float limit,
                      int32_t* ids, float* w, int32_t* counts, int32_t* basep, int32_t* row_tok,
                      int32_t* pos, uint16_t* h, float* d, float* y, uint32_t* ws,
                      int max_workgroups, void* stream) {
  const bool own_ws = ws == nullptr;

  if (!logits || !x || !w_gu || !w_dn || !ids || !w || !counts || !basep || !row_tok || !pos ||
      !h || !y || !w_gu->q || !w_gu->s || !w_dn->q || !w_dn->s || T < 1 || E < 1 ||
      k < 1 || k > E || k > MOE_MAX_K || max_workgroups < 0)
    return MOE_EINVAL;
  if (T > MOE_DECODE_MAX_T || E > MOE_MAX_E || k > MOE_DECODE_MAX_K) return MOE_ESHAPE;
  const int D = w_gu->K, N = w_gu->N, F = N / 2;
  if (w_gu->E != E || w_dn->E != E || N < 2 || (N & 1) || D < 32 || (D & 31) || w_dn->N != D ||
      w_dn->K != F || (F & 31))
    return MOE_ESHAPE;
  auto misaligned = [](const void* p) { return (((uintptr_t)p) & 15) != 0; };
  if (misaligned(x) || misaligned(h) || misaligned(w_gu->q) || misaligned(w_dn->q) ||
      misaligned(w_gu->s) || misaligned(w_dn->s) || (((uintptr_t)logits) & 3) ||
      (((uintptr_t)y) & 3) || (d && (((uintptr_t)d) & 3)) || (((uintptr_t)ws) & 3))
    return MOE_EALIGN;
  if ((int64_t)N * (D / 32) * 16 >= ((int64_t)1 << 31) ||
      (int64_t)D * (F / 32) * 16 >= ((int64_t)1 << 31))
    return MOE_ESHAPE;
  moe::LyArgs a{};
  int G = 0;
  size_t lds = 0;
  const int plan = moe::layer_plan(T, E, k, D, F, max_workgroups, &a, &G, &lds);
  if (plan < 0) return MOE_ELAUNCH;
  if (plan > 0)   // a shape the one-launch kernel does not take: the two launches
    return moe_launch_decode_two(logits, x, T, E, k, w_gu, w_dn, alpha, limit, ids, w, counts,
                                 basep, row_tok, pos, h, d, y, (hipStream_t)stream);
  a.logits = logits;
  a.x = x;
  a.gq = w_gu->q;
  a.gs = w_gu->s;
  a.gb = w_gu->bias;
  a.dq = w_dn->q;
  a.ds = w_dn->s;
  a.db = w_dn->bias;
  a.T = (int)T;
  a.E = E;
  a.k = k;
  a.D = D;
  a.F = F;
  a.N = N;
  a.alpha = alpha;
  a.limit = limit;
  a.ids = ids;
  a.w = w;
  a.counts = counts;
  a.basep = basep;
  a.row_tok = row_tok;
  a.pos = pos;
  a.h = h;
  a.d = d;
  a.y = y;
  if (own_ws) {
    ws = scratch_ptr();
    if (!ws) return MOE_ELAUNCH;
    moe::launch(fill_zero_u32, dim3(1), dim3(256), 0, (hipStream_t)stream, ws,
                (int)MOE_DECODE_WS_WORDS);
    if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
  }
  a.ws = ws;
  moe::launch(moe::decode_layer_kernel, dim3((unsigned)G), dim3(moe::kLyThreads), lds,
              (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

}  // namespace

extern "C" int mx4_moe_decode_persistent(const float* logits, const uint16_t* x, int64_t T, int E,
                                         int k, const mx4_experts* w_gu, const mx4_experts* w_dn,
                                         float alpha, float limit, int32_t* ids, float* w,
                                         int32_t* counts, int32_t* basep, int32_t* row_tok,
                                         int32_t* pos, uint16_t* h, float* d, float* y,
                                         uint32_t* ws, int max_workgroups, void* stream) {
  if (!ws) return MOE_EINVAL;
  return decode_persistent(logits, x, T, E, k, w_gu, w_dn, alpha, limit, ids, w, counts, basep,
                           row_tok, pos, h, d, y, ws, max_workgroups, stream);
}

extern "C" int mx4_moe_decode_persistent_static(const float* logits, const uint16_t* x, int64_t T,
                                                int E, int k, const mx4_experts* w_gu,
                                                const mx4_experts* w_dn, float alpha,
                                                float limit, int32_t* ids, float* w,
                                                int32_t* counts, int32_t* basep,
                                                int32_t* row_tok, int32_t* pos, uint16_t* h,
                                                float* d, float* y, int max_workgroups,
                                                void* stream) {
  return decode_persistent(logits, x, T, E, k, w_gu, w_dn, alpha, limit, ids, w, counts, basep,
                           row_tok, pos, h, d, y, nullptr, max_workgroups, stream);
}
