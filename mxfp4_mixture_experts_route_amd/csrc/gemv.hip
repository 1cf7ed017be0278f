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
//  * The wavefront finds its expert by itself (one load of counts[], a ballot) and then issues
//    every load of a K segment of up to 24 chunks at once (384 B of nibbles per lane; all of K
//    at gpt-oss shapes), scales first and nibbles in K order. Loads complete in issue order, so
//    chunk i is computed as soon as its own bytes arrive and the compute overlaps the stream.
//    A lane's scale for chunk c is byte g of dword c of its (16-byte padded) scale row, so 6
//    dwordx4 loads carry the scales of 24 chunks.
//  * All global loads are buffer loads with per-lane offsets computed once; lanes with nothing to
//    load point past the resource and read zeros.
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
constexpr int kGvSeg = 24;        // chunks per K segment, all in flight at once (K <= 3072: one)
constexpr int kGvPitch = 80;      // LDS bytes per staged 32-element block (64 used)
constexpr int kGvLdsBudget = 65536;
constexpr int kGvMaxStage = 6;    // 16-byte pieces per thread when all activation rows are staged
constexpr int kGvMaxThreads = 256;

// Expert of this wavefront's slot: the slot-th expert with a non-zero count, or -1. c64 is this
// lane's counts[lane] (0 past E), loaded by the caller before anything else; experts past 64
// are scanned 64 at a time. No LDS, no barrier.
__device__ __forceinline__ int wave_slot_expert(const int32_t* __restrict__ counts, int E,
                                                int slot, int c64) {
  const int lane = (int)(threadIdx.x & 63);
  int seen = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    const bool live = base == 0 ? (c64 > 0) : ((e < E) && (counts[e] > 0));
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

  // Vector loads complete in issue order, so they are issued in the order they are needed:
  // counts (expert lookup), the activations, the bias, then the weights.
  // 1. counts for the expert lookup, then the activations that do not depend on the CSR
  const int c64 = (lane < E) ? counts[lane] : 0;
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
  const int e = wave_slot_expert(counts, E, (int)blockIdx.y, c64);
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
  const int SP = scale_row_bytes(KB);
  const int wlast = KB - (C - 1) * kChunkBlocks;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + 16 * (size_t)e * N * KB, (uint32_t)N * KB * 16);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s + (size_t)e * N * SP, (uint32_t)N * SP);
  const uint32_t wo = valid ? ((uint32_t)n * kChunkBlocks + lg) * 16 : kOOB;       // full chunk
  const uint32_t wol = (valid && lg < wlast) ? ((uint32_t)n * wlast + lg) * 16 : kOOB;  // last
  const uint32_t so = valid ? (uint32_t)n * SP : kOOB;
  // branch-free: a chunk past K gets an out-of-range offset and reads zeros
  auto load_chunk = [&](int c, u32x4_t& wq) {
    const uint32_t off = (c < C - 1) ? wo : (c == C - 1 ? wol : kOOB);
    wq = buf_load16(rq, off, (uint32_t)c * N * (kChunkBlocks * 16));
  };
  // one K segment in K order: for every 4 chunks, their scale dwords, then their nibbles. The
  // scheduling barriers keep that issue order (the compiler would otherwise move the scale
  // loads last, and chunk 0 would then wait for the whole segment).
  u32x4_t wq[kGvSeg];
  uint32_t sc[kGvSeg];
  auto load_segment = [&](int c0) {
#pragma unroll
    for (int i = 0; i < kGvSeg / 4; ++i) {
      // 16 scale bytes = 4 chunks; a group past the padded scale row reads zeros (it would
      // otherwise read the next row's scales, where a NaN byte would poison 0 * scale)
      const uint32_t g_off = (uint32_t)(c0 + 4 * i) * 4;
      const u32x4_t v = buf_load16(rs, g_off < (uint32_t)SP ? so : kOOB, g_off);
      sc[4 * i + 0] = v[0];
      sc[4 * i + 1] = v[1];
      sc[4 * i + 2] = v[2];
      sc[4 * i + 3] = v[3];
#pragma unroll
      for (int k = 0; k < 4; ++k) load_chunk(c0 + 4 * i + k, wq[4 * i + k]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const float b0 = (valid && bias && lg == 0) ? bias[(size_t)e * N + n] : 0.0f;
  load_segment(0);

  const int cnt = counts[e];
  const int row0 = basep[e];

  // 4. activations staged up front go to LDS, followed by one all-zero block
  const size_t zero_blk = (size_t)(stage_all ? a_rows : rb) * KB;
  if (tid < 4) *reinterpret_cast<uint4*>(xs + zero_blk * kGvPitch + tid * 16) = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int i = 0; i < kGvMaxStage; ++i) {
    const int p = tid + i * nthreads;
    if (p < all_pieces)
      *reinterpret_cast<uint4*>(xs + (size_t)(p >> 2) * kGvPitch + (p & 3) * 16) = stage[i];
  }

  for (int p0 = 0; p0 < cnt; p0 += rb) {
    const int nr = min(rb, cnt - p0);

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

    for (int c0 = 0; c0 < C; c0 += kGvSeg) {
      if (c0 > 0 || p0 > 0) load_segment(c0);   // later segments / passes (K > 3072, > rb rows)
#pragma unroll
      for (int i = 0; i < kGvSeg; ++i) {
        // straight-line over the segment (no branches, so each chunk waits only for its own
        // loads): blocks past K read zero weights and the block's x is clamped, then dropped
        const int kb = (c0 + i) * kChunkBlocks + lg;
        const bool in_k = kb < KB;
        {
          const float scl = e8m0_scale_operand(__builtin_amdgcn_ubfe(sc[i], 8 * lg, 8));
          bf16x2_t wv[16];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            wv[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wq[i][d], scl, 0);
            wv[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wq[i][d], scl, 1);
            wv[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wq[i][d], scl, 2);
            wv[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wq[i][d], scl, 3);
          }
#pragma unroll
          for (int rr = 0; rr < kGvMaxRB; ++rr) {
            if (rr < nr) {
              // blocks past K (zero weights) read the zero block instead of activations
              const uint8_t* xp = xs + (in_k ? (size_t)xrow[rr] * KB + kb : zero_blk) * kGvPitch;
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xp + 16 * d);
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                  const uint32_t xw = xv[bb];
                  acc[rr] = __builtin_amdgcn_fdot2_f32_bf16(wv[4 * d + bb], as_bf16x2(xw),
                                                            acc[rr], false);
                }
              }
            }
          }
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
  int rb = (int)((moe::kGvLdsBudget - moe::kGvPitch) / row_lds);   // rows + the zero block
  if (rb > moe::kGvMaxRB) rb = moe::kGvMaxRB;
  if (rb < 1) return MOE_ESHAPE;
  const size_t lds = (stage_all ? (size_t)a_rows * row_lds : (size_t)rb * row_lds) + moe::kGvPitch;
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
