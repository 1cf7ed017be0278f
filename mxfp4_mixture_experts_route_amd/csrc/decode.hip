// mx4_moe_decode: the routed MXFP4 expert chain of a few tokens in two launches.
//
// Sources: PR #3579 "dasLLAMA gpt-oss arc", PR body section "Fused MoE expert chain" and the
// fused chain commit (stage 1: gate and up rows + bias + activation; stage 2: every routed
// expert's down row + bias and the routing-weighted sum in slot order), Metal fusion-lane commit
// (bias-seeded accumulators; the per-expert padded-prefix bases of the bucket pass); PR #3558
// section "gpt-oss: mx4 kernels to the lab-winning shape" (the routed-expert GEMV).
//
// At decode sizes every launch costs microseconds of ramp and drain, which at T = 1 is as much
// as the route, bucket and combine work itself. Here:
//  * Launch 1: every workgroup of routed row rho = t*k + s routes token t itself (its
//    wavefront 0: for E <= 64 the rank of every logit against the row staged in LDS, else k
//    rounds of arg-best over the E logits; the pick goes to the others through LDS), takes
//    pick s as its expert and runs the
//    gate_up projection + clamped SwiGLU-OAI for that row with the wavefront engine of
//    gemv_core.hpp; h is written in routed-row order. One extra workgroup writes the routing
//    (ids, w) and the CSR of tile 1 (counts, basep, row_tok, pos) for the caller.
//  * Launch 2: a workgroup owns 16 rows of the down projection of one token, with one wavefront
//    (or a K-split pair) per slot; the slots meet in LDS, where wavefront 0 adds bias-seeded d
//    rows into y in slot order, so d never has to leave the chip (it is written only when the
//    caller asks for it).
// An expert that several of the tokens picked is streamed once per pick, so this path is for
// T = 1 (or a few tokens); the CSR path (mx4_moe_gemv / mx4_moe_gemm) streams each expert once.
#include "gemv_core.hpp"
#include "launch.hpp"
#include "route_core.hpp"

namespace moe {

constexpr int kDecMaxThreads = 512;

// Launch 1, extra workgroup: routing of every token and the CSR with tile 1, for the caller.
__device__ __forceinline__ void decode_bookkeeping(const float* __restrict__ logits, int T, int E,
                                                int k, int32_t* __restrict__ ids,
                                                float* __restrict__ w, int32_t* __restrict__ counts,
                                                int32_t* __restrict__ basep,
                                                int32_t* __restrict__ row_tok,
                                                int32_t* __restrict__ pos) {
  __shared__ int sid[MOE_DECODE_MAX_T * MOE_DECODE_MAX_K];
  __shared__ int bp[MOE_MAX_E + 1];
  const int tid = (int)threadIdx.x, nthreads = (int)blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, waves = nthreads >> 6;
  const int R = T * k;
  for (int t = wave; t < T; t += waves) {
    int my_id;
    float my_v;
    wave_topk(logits + (size_t)t * E, E, k, my_id, my_v);
    write_topk(my_id, my_v, k, ids + t * k, w + t * k);
    if (lane < k) sid[t * k + lane] = my_id;
  }
  __syncthreads();
  for (int i = tid; i < E; i += nthreads) {
    int c = 0;
    for (int r = 0; r < R; ++r) c += (sid[r] == i);
    counts[i] = c;
    bp[i] = c;
  }
  __syncthreads();
  if (wave == 0) {   // exclusive prefix of the counts (tile 1: no padding)
    int carry = 0;
    for (int base = 0; base < E; base += 64) {
      const int i = base + lane;
      const int c = i < E ? bp[i] : 0;
      int v = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
      }
      if (i < E) bp[i] = carry + v - c;
      carry += __shfl(v, 63);
    }
    if (lane == 0) bp[E] = carry;
  }
  __syncthreads();
  for (int i = tid; i <= E; i += nthreads) basep[i] = bp[i];
  for (int r = tid; r < R; r += nthreads) {
    // CSR row of (t, s): after every earlier token routed to the same expert
    const int e = sid[r], t = r / k;
    int rank = 0;
    for (int r2 = 0; r2 < t * k; ++r2) rank += (sid[r2] == e);
    const int p = bp[e] + rank;
    pos[r] = p;
    row_tok[p] = t;
  }
}

// Gate_up + SwiGLU-OAI of routed row rho for the units [ubase, ubase + waves / ksplit) of 8 h
// columns (gate rows j..j+7 and the matching up rows) each, K split over ksplit wavefronts.
// Routes token rho / k itself.
template <int SEG>
__device__ __forceinline__ void gate_up_item(const float* __restrict__ logits,
                                             const uint16_t* __restrict__ x, int E, int k,
                                             const uint8_t* __restrict__ q,
                                             const uint8_t* __restrict__ s,
                                             const float* __restrict__ bias, int N, int K,
                                             float alpha, float limit, int ksplit, int rho,
                                             int ubase, uint16_t* __restrict__ h, uint8_t* xs) {
  const int KB = K >> 5;
  const int C = (KB + kChunkBlocks - 1) / kChunkBlocks;
  const int tid = (int)threadIdx.x;
  const int nthreads = (int)blockDim.x;
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
  const int F = N >> 1;
  const int t = rho / k, slot = rho - t * k;
  const uint32_t row_bytes = (uint32_t)K * 2;

  // 1. token t's activation row copied to LDS (LDS-DMA), then routing: the workgroup's expert is
  // pick `slot` of the token's top-k. Wavefront 0 alone routes and leaves the pick in LDS (in the
  // spare bytes of its own K-part slot, which it never writes: it holds part 0): every wavefront
  // would compute the same pick. For E <= 64 the logits row comes by LDS-DMA too, right after
  // the copy, so one wait lands both, and the rank reads it from LDS.
  lds_dma_copy(x + (size_t)t * K, row_bytes, xs, wave, nthreads >> 6);
  const size_t zoff = ((size_t)row_bytes + 1023) & ~(size_t)1023;
  // LDS after the row: a zero block, then 1 KB per wavefront (K-part sums)
  if (tid < 4) *reinterpret_cast<uint4*>(xs + zoff + tid * 16) = make_uint4(0u, 0u, 0u, 0u);
  __builtin_amdgcn_sched_barrier(0);
  // wavefront 0's 1 KB: the logits row, the rank keys at +256, the pick at +768
  uint8_t* const slot0 = xs + zoff + 64;
  int* const pick = reinterpret_cast<int*>(slot0 + 768);
  if (wave == 0) {
    int e0;
    if (E <= kWave) {   // one logit per lane: rank against the row in LDS
      float* lrow = reinterpret_cast<float*>(slot0);
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(logits + (size_t)t * E, (uint32_t)E * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rl, (__attribute__((address_space(3))) void*)lrow, 4, (uint32_t)lane * 4, 0, 0, 0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      // lrow: 0 past E (read past the resource)
      e0 = rank_pick(wave_rank_lds(lrow, reinterpret_cast<uint64_t*>(slot0 + 256), E), slot);
    } else {
      int my_id;
      float my_v;
      wave_topk(logits + (size_t)t * E, E, k, my_id, my_v);
      e0 = __shfl(my_id, slot);
    }
    if (lane == 0) *pick = e0;
  }
  // every wavefront's share of the row copy has landed; the pick and the zero block are written
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  // the top-k order is total (route_core.hpp), so the pick is an expert of [0, E) whatever the
  // logits hold; it is clamped all the same, as an id outside would address memory outside the
  // weight stack
  const int e = min(max(*pick, 0), E - 1);

  // 2. 16 rows (gate rows j..j+7 and the matching up rows) and a part of K per wavefront
  const int part = wave % ksplit;
  const int unit = ubase + wave / ksplit;
  int cb, ce, Cp;
  k_part_range(C, part, ksplit, cb, ce, Cp);
  auto row_of = [&](int r16, bool& ok) {
    const int jj = unit * 8 + (r16 & 7);
    ok = jj < F;
    return r16 < 8 ? jj : F + jj;
  };
  bool valid;
  const int n = row_of(lr, valid);
  Mx4Wave<SEG> ws;
  ws.init(q, s, e, n, valid, N, K, ce);
  // bias seeds (gate rows j..j+7, up rows F+j..F+j+7; F % 8 == 0, so a unit is whole or past F)
  float b4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int ju = __builtin_amdgcn_readfirstlane(unit * 8);
  const int eu = __builtin_amdgcn_readfirstlane(e);
  if (bias && part == 0 && ju < F)
    scalar_seed16(bias + (size_t)eu * N + ju, bias + (size_t)eu * N + F + ju, b4);
  ws.load_segment(cb);

  // 3. the zero block after the staged row, then the partial sums of the K parts (all written
  // or landed before the barrier above: the chunks run as their bytes arrive)
  const uint8_t* xzero = xs + zoff;
  f32x4_t* red = reinterpret_cast<f32x4_t*>(xs + zoff + 64);

  // 4. one B column (the token); K segments; K parts meet in LDS
  f32x4_t acc = {b4[0], b4[1], b4[2], b4[3]};
  f32x4_t acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = cb; c0 < ce; c0 += SEG) {
    if (c0 > cb) ws.load_segment(c0);
    ws.run_segment(c0, KB, xs, xzero, lr == 0, acc, acc1);
  }
  acc += acc1;
  if (ksplit > 1) {
    if (part > 0) red[wave * 64 + lane] = acc;
    __syncthreads();
    if (part == 0)
      for (int pp = 1; pp < ksplit; ++pp) acc += red[(wave + pp) * 64 + lane];
  }

  // 5. SwiGLU-OAI: lanes 0 and 16 hold gate rows 0-3 / 4-7, lanes 32 and 48 the matching up rows
  if (part == 0) {
    float up[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) up[i] = __shfl_xor(acc[i], 32);
    if (lr == 0 && lg < 2) {
      const int j0 = unit * 8 + 4 * lg;
      uint32_t hb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hb[i] = f32_to_bf16_bits(swiglu_oai(acc[i], up[i], alpha, limit));
      uint16_t* dst = h + (size_t)rho * F + j0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j0 + i < F) dst[i] = (uint16_t)hb[i];
    }
  }
}

template <int SEG>
__global__ void __launch_bounds__(kDecMaxThreads)
decode_gate_up_kernel(const float* __restrict__ logits, const uint16_t* __restrict__ x, int T,
                      int E, int k, const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                      const float* __restrict__ bias, int N, int K, float alpha, float limit,
                      int ksplit, int32_t* __restrict__ ids, float* __restrict__ w,
                      int32_t* __restrict__ counts, int32_t* __restrict__ basep,
                      int32_t* __restrict__ row_tok, int32_t* __restrict__ pos,
                      uint16_t* __restrict__ h, int gx) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  // block 0 (dispatched first, so it never waits for a slot behind the items): the routing and
  // the CSR for the caller; blocks 1..: the items, gx a routed row
  if (blockIdx.x == 0) {
    decode_bookkeeping(logits, T, E, k, ids, w, counts, basep, row_tok, pos);
    return;
  }
  const int item = (int)blockIdx.x - 1;
  const int rho = item / gx, bx = item - rho * gx;
  const int upw = ((int)blockDim.x >> 6) / ksplit;
  gate_up_item<SEG>(logits, x, E, k, q, s, bias, N, K, alpha, limit, ksplit, rho, bx * upw, h,
                    xs);
}

template <int SEG>
__global__ void __launch_bounds__(kDecMaxThreads)
decode_down_kernel(const uint16_t* __restrict__ h, int E, int k, const int32_t* __restrict__ ids,
                   const float* __restrict__ w, const uint8_t* __restrict__ q,
                   const uint8_t* __restrict__ s, const float* __restrict__ bias, int D, int F,
                   int ksplit, float* __restrict__ d, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  const int KB = F >> 5;
  const int C = (KB + kChunkBlocks - 1) / kChunkBlocks;
  const int tid = (int)threadIdx.x;
  const int nthreads = (int)blockDim.x;
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
  const int t = (int)blockIdx.y, unit = (int)blockIdx.x;
  const uint32_t row_bytes = (uint32_t)F * 2;

  // 1. the token's k rows of h (routed-row order: slot s is row t*k + s) to LDS, and this
  // wavefront's slot and expert. The expert id comes through the scalar cache, counted apart
  // from the copy: the weights go out as soon as it arrives (a vector load of it was waited for
  // together with the whole copy, whose trip count the compiler does not know)
  const int slot = __builtin_amdgcn_readfirstlane(wave / ksplit), part = wave % ksplit;
  const int e = min(max(((const __attribute__((address_space(4))) int32_t*)ids)[t * k + slot], 0),
                    E - 1);   // in [0, E) by the routing; clamped as in launch 1
  lds_dma_copy(h + (size_t)t * k * F, (uint32_t)k * row_bytes, xs, wave, nthreads >> 6);
  __builtin_amdgcn_sched_barrier(0);
  int cb, ce, Cp;
  k_part_range(C, part, ksplit, cb, ce, Cp);
  const int n = unit * 16 + lr;
  Mx4Wave<SEG> ws;
  ws.init(q, s, e, n, n < D, D, F, ce);
  // bias seeds (rows unit*16..+15 are all inside D: D % 16 == 0)
  float b4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (bias && part == 0) {
    const float* br = bias + (size_t)__builtin_amdgcn_readfirstlane(e) * D + unit * 16;
    scalar_seed16(br, br + 8, b4);
  }
  ws.load_segment(cb);

  const size_t zero_off = ((size_t)k * row_bytes + 1023) & ~(size_t)1023;
  if (tid < 4) *reinterpret_cast<uint4*>(xs + zero_off + tid * 16) = make_uint4(0u, 0u, 0u, 0u);
  const uint8_t* xzero = xs + zero_off;
  f32x4_t* red = reinterpret_cast<f32x4_t*>(xs + zero_off + 64);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(SEG + SEG / 4));   // the LDS-DMA copy has landed
  __syncthreads();

  f32x4_t acc = {b4[0], b4[1], b4[2], b4[3]};
  f32x4_t acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = cb; c0 < ce; c0 += SEG) {
    if (c0 > cb) ws.load_segment(c0);
    ws.run_segment(c0, KB, xs + (size_t)slot * row_bytes, xzero, lr == 0, acc, acc1);
  }
  acc += acc1;

  // 2. every wavefront's partial rows meet in LDS; wavefront 0 forms d of each slot (parts in
  // order, bias in part 0) and y = sum over slots, in slot order, of w * d
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  float yv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int sl = 0; sl < k; ++sl) {
    f32x4_t ds = red[(sl * ksplit) * 64 + lane];
    for (int pp = 1; pp < ksplit; ++pp) ds += red[(sl * ksplit + pp) * 64 + lane];
    const float ws_w = w[t * k + sl];
#pragma unroll
    for (int i = 0; i < 4; ++i) yv[i] = fmaf(ws_w, ds[i], yv[i]);
    if (d && lr == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nn = unit * 16 + 4 * lg + i;
        if (nn < D) d[((size_t)t * k + sl) * D + nn] = ds[i];
      }
    }
  }
  if (lr == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nn = unit * 16 + 4 * lg + i;
      if (nn < D) y[(size_t)t * D + nn] = yv[i];
    }
  }
}

}  // namespace moe

int moe_launch_decode_two(const float* logits, const uint16_t* x, int64_t T, int E, int k,
                          const mx4_experts* w_gu, const mx4_experts* w_dn, float alpha,
                          float limit, int32_t* ids, float* w, int32_t* counts, int32_t* basep,
                          int32_t* row_tok, int32_t* pos, uint16_t* h, float* d, float* y,
                          hipStream_t stream);

extern "C" int mx4_moe_decode(const float* logits, const uint16_t* x, int64_t T, int E, int k,
                              const mx4_experts* w_gu, const mx4_experts* w_dn, float alpha,
                              float limit, int32_t* ids, float* w, int32_t* counts,
                              int32_t* basep, int32_t* row_tok, int32_t* pos, uint16_t* h,
                              float* d, float* y, void* stream) {
  if (!logits || !x || !w_gu || !w_dn || !ids || !w || !counts || !basep || !row_tok || !pos ||
      !h || !y || !w_gu->q || !w_gu->s || !w_dn->q || !w_dn->s || T < 1 || E < 1 || k < 1 ||
      k > E || k > MOE_MAX_K)
    return MOE_EINVAL;
  if (T > MOE_DECODE_MAX_T || E > MOE_MAX_E || k > MOE_DECODE_MAX_K) return MOE_ESHAPE;
  const int D = w_gu->K, N = w_gu->N, F = N / 2;
  if (w_gu->E != E || w_dn->E != E || N < 2 || (N & 1) || D < 32 || (D & 31) || w_dn->N != D ||
      w_dn->K != F || (F & 31))
    return MOE_ESHAPE;
  auto misaligned = [](const void* p) { return (((uintptr_t)p) & 15) != 0; };
  if (misaligned(x) || misaligned(h) || misaligned(w_gu->q) || misaligned(w_dn->q) ||
      misaligned(w_gu->s) || misaligned(w_dn->s) || (((uintptr_t)logits) & 3) ||
      (((uintptr_t)y) & 3) || (d && (((uintptr_t)d) & 3)))
    return MOE_EALIGN;
  return moe_launch_decode_two(logits, x, T, E, k, w_gu, w_dn, alpha, limit, ids, w, counts,
                               basep, row_tok, pos, h, d, y, (hipStream_t)stream);
}

// The two launches of mx4_moe_decode (arguments already checked); also what
// mx4_moe_decode_persistent runs for shapes its one-launch kernel does not take.
int moe_launch_decode_two(const float* logits, const uint16_t* x, int64_t T, int E, int k,
                          const mx4_experts* w_gu, const mx4_experts* w_dn, float alpha,
                          float limit, int32_t* ids, float* w, int32_t* counts, int32_t* basep,
                          int32_t* row_tok, int32_t* pos, uint16_t* h, float* d, float* y,
                          hipStream_t st) {
  const int D = w_gu->K, N = w_gu->N, F = N / 2;
  const int C1 = (D / 32 + moe::kChunkBlocks - 1) / moe::kChunkBlocks;
  const int C2 = (F / 32 + moe::kChunkBlocks - 1) / moe::kChunkBlocks;
  const int R = (int)T * k;

  // launch 1: workgroups of ksplit * (1, 2 or 4 row groups) wavefronts, grid (units, R + 1)
  const int ks1 = moe::gv_ksplit(C1);
  const int units1 = (F + 7) / 8;
  const int64_t waves_total = (int64_t)units1 * R * ks1;
  int upw1 = 256 / 64 / ks1;
  while (upw1 > 1 && waves_total / (upw1 * ks1) < 640) upw1 >>= 1;
  const int waves1 = upw1 * ks1;
  // x row, zero block, then 1 KB per wavefront: K-part sums, and first each wavefront's copy of
  // the logits row (E <= 64)
  const size_t lds1 = (((size_t)D * 2 + 1023) & ~(size_t)1023) + 64 + (size_t)waves1 * 64 * 16;
  // launch 2: one workgroup per (16 rows, token), ksplit wavefronts per slot
  int ks2 = moe::gv_ksplit(C2);
  while (ks2 > 1 && k * ks2 * 64 > moe::kDecMaxThreads) --ks2;
  const int waves2 = k * ks2;
  const size_t lds2 = (((size_t)k * F * 2 + 1023) & ~(size_t)1023) + 64 + (size_t)waves2 * 64 * 16;
  if (lds1 > 65536 || lds2 > 65536 || 64 * waves2 > moe::kDecMaxThreads) return MOE_ESHAPE;
  // 32-bit buffer offsets
  if ((int64_t)N * (D / 32) * 16 >= ((int64_t)1 << 31) ||
      (int64_t)D * (F / 32) * 16 >= ((int64_t)1 << 31))
    return MOE_ESHAPE;

  const int gx1 = (units1 + upw1 - 1) / upw1;
  const dim3 g1((unsigned)(1 + gx1 * R));
  moe::launch(moe::decode_gate_up_kernel<moe::kGvSeg>, g1, dim3(64 * waves1), lds1, st, logits, x,
              (int)T, E, k, w_gu->q, w_gu->s, w_gu->bias, N, D, alpha, limit, ks1, ids, w, counts,
              basep, row_tok, pos, h, gx1);
  if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
  const dim3 g2((unsigned)((D + 15) / 16), (unsigned)T);
  moe::launch(moe::decode_down_kernel<moe::kGvSeg>, g2, dim3(64 * waves2), lds2, st, h, E, k, ids, w,
              w_dn->q, w_dn->s, w_dn->bias, D, F, ks2, d, y);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
