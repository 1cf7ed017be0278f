// mx4_moe_gemv: routed-expert MXFP4 projection for decode (a handful of rows per expert).
//
// Sources: PR #3558 "dasLLAMA: dig the last two board reds green", section "gpt-oss: mx4 kernels
// to the lab-winning shape" and its ladder table (the routed-expert GEMV at gpt-oss shape: load
// every weight byte exactly once, decode e2m1 through a 16-entry table and the e8m0 exponent
// arithmetically instead of through a dependent table load); PR #3579 "dasLLAMA gpt-oss arc",
// Metal fusion-lane commit (accumulators start from the expert's bias row; the SwiGLU-OAI
// epilogue leaves rows that are not live untouched) and fused MoE chain commit (gate and up rows
// + bias + activation in one stage).
//
// gfx950 mapping. Bound by HBM; at decode sizes (tens of MB per launch) the time goes to memory
// latency, so every weight load of a wavefront is in flight before it computes anything.
//  * Weights are in the chunked layout (chunks of 4 MX blocks, all rows of a chunk together). A
//    wavefront owns 16 weight rows: lane (r = lane%16, g = lane/16) takes block g of every chunk
//    of row r, so each load instruction of the wavefront reads one contiguous 1 KB run.
//  * The wavefront finds its expert by itself (one load of counts[], a ballot) and then issues the
//    loads of its first 16 chunks at once (256 B per lane); each ring slot is refilled with the
//    chunk 16 ahead as soon as it is consumed, so a launch waits for HBM latency about once.
//  * When every activation row fits (decode: a_rows * K * 2 bytes <= 24 KB) the workgroup stages
//    them all into LDS at kernel start, independently of the CSR; otherwise it stages the
//    expert's rows per pass of up to 4 rows.
//  * e2m1 nibbles are decoded by v_cvt_scalef32_pk_bf16_fp4 (the CDNA4 hardware table: two codes
//    to two bf16 per instruction, with the block's e8m0 scale folded in; exact, since a scaled
//    e2m1 value has at most 2 significant bits) and multiplied with the bf16 activations by
//    v_dot2_f32_bf16 (exact products, fp32 sums). The e8m0 byte becomes the fp32 scale with
//    integer ops: no scale table, no dependent table load.
//  * The 4 lanes of a row are summed with two shuffles. In SwiGLU mode lanes 0-7 of a 16-row
//    group hold gate rows and lanes 8-15 the matching up rows, so one more shuffle pairs them.
#include "common.hpp"

namespace moe {

constexpr int kGvMaxRB = 4;       // activation rows per pass (per-expert staging)
constexpr int kGvRing = 16;       // chunk loads in flight per lane (a ring refilled as it drains)
constexpr int kGvPitch = 80;      // LDS bytes per staged 32-element block (64 used)
constexpr int kGvLdsBudget = 65536;
constexpr int kGvMaxStage = 6;    // 16-byte pieces per thread when all activation rows are staged
constexpr int kGvMaxThreads = 256;

// Expert of this wavefront's slot: the slot-th expert with a non-zero count, or -1. One load of
// counts[] per 64 experts and a ballot; no LDS, no barrier.
__device__ __forceinline__ int wave_slot_expert(const int32_t* __restrict__ counts, int E,
                                                int slot) {
  const int lane = (int)(threadIdx.x & 63);
  int seen = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    const bool live = (e < E) && (counts[e] > 0);
    uint64_t ballot = __ballot(live);
    const int n = __popcll(ballot);
    if (slot < seen + n) {
      for (int i = seen; i < slot; ++i) ballot &= ballot - 1;   // drop lower live experts
      return base + __ffsll((unsigned long long)ballot) - 1;
    }
    seen += n;
  }
  return -1;
}

template <int ACT>
__global__ void __launch_bounds__(kGvMaxThreads, 2)
gemv_kernel(const uint16_t* __restrict__ a, const int32_t* __restrict__ a_row, int a_rows,
            const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
            const float* __restrict__ bias, const int32_t* __restrict__ counts,
            const int32_t* __restrict__ basep, int E, int N, int K, float alpha, float limit,
            void* __restrict__ out, int rb, int stage_all) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  constexpr bool swiglu = (ACT == MOE_ACT_SWIGLU_OAI);
  const int KB = K >> 5;
  const int C = (KB + kChunkBlocks - 1) / kChunkBlocks;
  const int tid = (int)threadIdx.x;
  const int nthreads = (int)blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int F = N >> 1;

  // 1. activations that do not depend on the CSR: issue their loads first
  const int all_pieces = stage_all ? a_rows * KB * 4 : 0;
  uint4 stage[kGvMaxStage];
#pragma unroll
  for (int i = 0; i < kGvMaxStage; ++i) {
    const int p = tid + i * nthreads;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (p < all_pieces) v = *reinterpret_cast<const uint4*>(a + (size_t)p * 8);
    stage[i] = v;
  }

  // 2. expert of this workgroup's slot (each wavefront on its own)
  const int e = wave_slot_expert(counts, E, (int)blockIdx.y);
  if (e < 0) return;  // uniform over the workgroup: fewer live experts than slots

  // 3. this wavefront's 16 weight rows
  const int unit = (int)blockIdx.x * (nthreads >> 6) + wave;
  int n, j = 0;
  bool valid;
  if (swiglu) {
    j = unit * 8 + (lr & 7);
    valid = j < F;
    n = (lr < 8) ? j : F + j;
  } else {
    n = unit * 16 + lr;
    valid = n < N;
  }
  const size_t ebase = (size_t)e * N * KB;
  auto load_chunk = [&](int c, u32x4_t& wq, uint32_t& ex) {
    const int kb = c * kChunkBlocks + lg;
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    uint32_t x = 127u;
    if (valid && c < C && kb < KB) {
      const int w = min(kChunkBlocks, KB - c * kChunkBlocks);
      const size_t blk = ebase + (size_t)c * N * kChunkBlocks + (size_t)n * w + lg;
      v = *reinterpret_cast<const u32x4_t*>(q + 16 * blk);
      x = s[blk];
    }
    wq = v;
    ex = x;
  };
  u32x4_t wq[kGvRing];
  uint32_t ex[kGvRing];
#pragma unroll
  for (int i = 0; i < kGvRing; ++i) load_chunk(i, wq[i], ex[i]);

  const int cnt = counts[e];
  const int row0 = basep[e];
  const float b0 = (valid && bias && lg == 0) ? bias[(size_t)e * N + n] : 0.0f;

  // 4. activations staged up front go to LDS
#pragma unroll
  for (int i = 0; i < kGvMaxStage; ++i) {
    const int p = tid + i * nthreads;
    if (p < all_pieces)
      *reinterpret_cast<uint4*>(xs + (size_t)(p >> 2) * kGvPitch + (p & 3) * 16) = stage[i];
  }

  for (int p0 = 0; p0 < cnt; p0 += rb) {
    const int nr = min(rb, cnt - p0);
    if (p0 > 0) {   // another pass over the same rows (more than rb rows): refill the ring
#pragma unroll
      for (int i = 0; i < kGvRing; ++i) load_chunk(i, wq[i], ex[i]);
    }
    if (!stage_all) {
      __syncthreads();  // the previous pass is done with xs
      for (int p = tid; p < nr * KB * 4; p += nthreads) {
        const int rr = p / (KB * 4);
        const int rem = p - rr * KB * 4;
        const int r = row0 + p0 + rr;
        const int64_t src = a_row ? (int64_t)a_row[r] : (int64_t)r;
        const uint4 v = *reinterpret_cast<const uint4*>(a + src * K + rem * 8);
        *reinterpret_cast<uint4*>(xs + ((size_t)rr * KB + (rem >> 2)) * kGvPitch + (rem & 3) * 16) = v;
      }
    }
    __syncthreads();
    // LDS row of each activation row of this pass
    int xrow[kGvMaxRB];
#pragma unroll
    for (int rr = 0; rr < kGvMaxRB; ++rr) {
      const int r = row0 + p0 + rr;
      xrow[rr] = !stage_all ? rr : (rr < nr ? (a_row ? a_row[r] : r) : 0);
    }
    float acc[kGvMaxRB];
#pragma unroll
    for (int rr = 0; rr < kGvMaxRB; ++rr) acc[rr] = b0;  // bias-seeded accumulator

    for (int c0 = 0; c0 < C; c0 += kGvRing) {
#pragma unroll
      for (int i = 0; i < kGvRing; ++i) {
        const int c = c0 + i;
        const int kb = c * kChunkBlocks + lg;
        if (c < C) {
          if (kb < KB) {
            const float sc = e8m0_to_f32(ex[i]);
            bf16x2_t wv[16];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              wv[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wq[i][d], sc, 0);
              wv[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wq[i][d], sc, 1);
              wv[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wq[i][d], sc, 2);
              wv[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wq[i][d], sc, 3);
            }
#pragma unroll
            for (int rr = 0; rr < kGvMaxRB; ++rr) {
              if (rr < nr) {
                const uint8_t* xp = xs + ((size_t)xrow[rr] * KB + kb) * kGvPitch;
                float part = 0.0f;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                  const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xp + 16 * d);
#pragma unroll
                  for (int bb = 0; bb < 4; ++bb) {
                    const uint32_t xw = xv[bb];
                    part = __builtin_amdgcn_fdot2_f32_bf16(wv[4 * d + bb], as_bf16x2(xw), part,
                                                           false);
                  }
                }
                acc[rr] += part;
              }
            }
          }
          load_chunk(c + kGvRing, wq[i], ex[i]);   // refill the slot (no load past K)
        }
      }
    }

#pragma unroll
    for (int rr = 0; rr < kGvMaxRB; ++rr) {
      if (rr < nr) {
        float g = acc[rr];
        g += __shfl_xor(g, 16);
        g += __shfl_xor(g, 32);
        const int r = row0 + p0 + rr;
        if (swiglu) {
          const float up = __shfl_xor(g, 8);
          if (lr < 8 && lg == 0 && valid) {
            const float h = swiglu_oai(g, up, alpha, limit);
            reinterpret_cast<uint16_t*>(out)[(size_t)r * F + j] = (uint16_t)f32_to_bf16_bits(h);
          }
        } else if (lg == 0 && valid) {
          reinterpret_cast<float*>(out)[(size_t)r * N + n] = g;
        }
      }
    }
  }
}

}  // namespace moe

// Host launcher shared with the C ABI entry point (argument checks are done by the caller).
int moe_launch_gemv(const uint16_t* a, const int32_t* a_row, int64_t a_rows, const mx4_experts* w,
                    const int32_t* counts, const int32_t* basep, int tile_m, int64_t mpad_max,
                    int act, float alpha, float limit, void* out, hipStream_t stream) {
  const int KB = w->K / 32;
  const size_t row_lds = (size_t)KB * moe::kGvPitch;
  const int units = (act == MOE_ACT_SWIGLU_OAI) ? (w->N / 2 + 7) / 8 : (w->N + 15) / 16;
  int64_t slots = mpad_max / tile_m;
  if (slots > w->E) slots = w->E;
  // 4 wavefronts per workgroup: enough threads to stage every activation row up front
  const int waves = 4;
  const int threads = 64 * waves;
  const int stage_all =
      ((int64_t)a_rows * KB * 4 <= (int64_t)moe::kGvMaxStage * threads) ? 1 : 0;
  int rb = (int)(moe::kGvLdsBudget / row_lds);
  if (rb > moe::kGvMaxRB) rb = moe::kGvMaxRB;
  if (rb < 1) return MOE_ESHAPE;
  const size_t lds = stage_all ? (size_t)a_rows * row_lds : (size_t)rb * row_lds;
  const int64_t bx = (units + waves - 1) / waves;
  if (act == MOE_ACT_SWIGLU_OAI)
    hipLaunchKernelGGL(moe::gemv_kernel<MOE_ACT_SWIGLU_OAI>, dim3((unsigned)bx, (unsigned)slots),
                       dim3(threads), lds, stream, a, a_row, (int)a_rows, w->q, w->s, w->bias,
                       counts, basep, w->E, w->N, w->K, alpha, limit, out, rb, stage_all);
  else
    hipLaunchKernelGGL(moe::gemv_kernel<MOE_ACT_NONE>, dim3((unsigned)bx, (unsigned)slots),
                       dim3(threads), lds, stream, a, a_row, (int)a_rows, w->q, w->s, w->bias,
                       counts, basep, w->E, w->N, w->K, alpha, limit, out, rb, stage_all);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
