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
// gfx950 mapping. The kernel is bound by HBM: every weight byte is read once, in 256-byte runs.
//  * A wavefront works on 4 weight rows at a time, 16 lanes per row; lane `sub` of a row takes the
//    32-element MX blocks sub, sub+16, sub+32, ... so each 16-lane group reads 256 contiguous
//    bytes per load and the 4 groups cover 4 rows.
//  * e2m1 nibbles are decoded by v_cvt_scalef32_pk_bf16_fp4 (the CDNA4 hardware table: two codes
//    to two bf16 per instruction, with the block's e8m0 scale folded in; exact, since a scaled
//    e2m1 value has at most 2 significant bits) and multiplied with the bf16 activations by
//    v_dot2_f32_bf16 (exact products, fp32 sums). The e8m0 byte becomes the fp32 scale with
//    integer ops, so there is no scale table and no dependent table load.
//  * The activation rows of the expert are staged once per workgroup in LDS (80-byte pitch per
//    block, which keeps the 16 lanes of a row group on distinct banks).
//  * A 16-lane butterfly reduces each row; SwiGLU mode puts the gate row in lanes 0-31 and its
//    up row 32 lanes higher, so one cross-half shuffle pairs them for the epilogue.
#include "common.hpp"

namespace moe {

constexpr int kGvThreads = 256;   // 4 wavefronts
constexpr int kGvMaxRB = 4;       // activation rows per pass
constexpr int kGvUnroll = 6;      // blocks in flight per lane per iteration
constexpr int kGvPitch = 80;      // LDS bytes per staged 32-element block (64 used)
constexpr int kGvLdsBudget = 65536;

__global__ void __launch_bounds__(kGvThreads)
gemv_kernel(const uint16_t* __restrict__ a, const int32_t* __restrict__ a_row,
            const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
            const float* __restrict__ bias, const int32_t* __restrict__ counts,
            const int32_t* __restrict__ basep, int E, int N, int K, int act, float alpha,
            float limit, void* __restrict__ out, int rb, int units_per_wave) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  __shared__ int scratch[2];
  const int e = slot_expert(counts, E, (int)blockIdx.y, scratch);
  if (e < 0) return;  // fewer live experts than slots
  const int cnt = counts[e];
  const int row0 = basep[e];
  const int KB = K >> 5;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, grp = lane >> 4, sub = lane & 15;
  const bool swiglu = (act == MOE_ACT_SWIGLU_OAI);
  const int F = N >> 1;
  const size_t row_bytes = (size_t)K >> 1;
  const uint8_t* qe = q + (size_t)e * N * row_bytes;
  const uint8_t* se = s + (size_t)e * N * KB;

  for (int p0 = 0; p0 < cnt; p0 += rb) {
    const int nr = min(rb, cnt - p0);
    // stage nr activation rows: 16-byte pieces, 4 per block
    const int pieces = nr * KB * 4;
    for (int p = tid; p < pieces; p += kGvThreads) {
      const int rr = p / (KB * 4);
      const int rem = p - rr * KB * 4;
      const int r = row0 + p0 + rr;
      const int64_t src = a_row ? (int64_t)a_row[r] : (int64_t)r;
      const uint4 v = *reinterpret_cast<const uint4*>(a + src * K + rem * 8);
      *reinterpret_cast<uint4*>(xs + ((size_t)rr * KB + (rem >> 2)) * kGvPitch + (rem & 3) * 16) = v;
    }
    __syncthreads();

    for (int it = 0; it < units_per_wave; ++it) {
      const int u = ((int)blockIdx.x * units_per_wave + it) * 4 + wave;
      int n, j = 0;
      bool valid;
      if (swiglu) {
        j = 2 * u + (grp & 1);
        valid = j < F;
        n = (grp < 2) ? j : F + j;
      } else {
        n = 4 * u + grp;
        valid = n < N;
      }
      float acc[kGvMaxRB];
      const float b0 = (valid && bias && sub == 0) ? bias[(size_t)e * N + n] : 0.0f;
#pragma unroll
      for (int rr = 0; rr < kGvMaxRB; ++rr) acc[rr] = b0;  // bias-seeded accumulator

      const uint8_t* qrow = qe + (size_t)n * row_bytes;
      const uint8_t* srow = se + (size_t)n * KB;
      for (int kb0 = 0; kb0 < KB; kb0 += 16 * kGvUnroll) {
        u32x4_t wq[kGvUnroll];
        uint32_t ex[kGvUnroll];
#pragma unroll
        for (int jj = 0; jj < kGvUnroll; ++jj) {
          const int kb = kb0 + sub + 16 * jj;
          if (valid && kb < KB) {
            wq[jj] = *reinterpret_cast<const u32x4_t*>(qrow + (size_t)kb * 16);
            ex[jj] = srow[kb];
          } else {
            wq[jj] = u32x4_t{0u, 0u, 0u, 0u};
            ex[jj] = 127u;
          }
        }
#pragma unroll
        for (int jj = 0; jj < kGvUnroll; ++jj) {
          const int kb = kb0 + sub + 16 * jj;
          if (kb < KB) {
            const float sc = e8m0_to_f32(ex[jj]);
            bf16x2_t wv[16];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              wv[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wq[jj][d], sc, 0);
              wv[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wq[jj][d], sc, 1);
              wv[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wq[jj][d], sc, 2);
              wv[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wq[jj][d], sc, 3);
            }
#pragma unroll
            for (int rr = 0; rr < kGvMaxRB; ++rr) {
              if (rr < nr) {
                const uint8_t* xb = xs + ((size_t)rr * KB + kb) * kGvPitch;
                float part = 0.0f;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                  const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xb + 16 * d);
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
        }
      }

#pragma unroll
      for (int rr = 0; rr < kGvMaxRB; ++rr) {
        if (rr < nr) {
          const float g = row16_sum(acc[rr]);
          const int r = row0 + p0 + rr;
          if (swiglu) {
            const float up = __shfl_xor(g, 32);
            if (grp < 2 && sub == 0 && valid) {
              const float h = swiglu_oai(g, up, alpha, limit);
              reinterpret_cast<uint16_t*>(out)[(size_t)r * F + j] = (uint16_t)f32_to_bf16_bits(h);
            }
          } else if (sub == 0 && valid) {
            reinterpret_cast<float*>(out)[(size_t)r * N + n] = g;
          }
        }
      }
    }
    __syncthreads();  // the next pass restages xs
  }
}

}  // namespace moe

// Host launcher shared with the C ABI entry point (argument checks are done by the caller).
int moe_launch_gemv(const uint16_t* a, const int32_t* a_row, const mx4_experts* w,
                    const int32_t* counts, const int32_t* basep, int tile_m, int64_t mpad_max,
                    int act, float alpha, float limit, void* out, hipStream_t stream) {
  const int KB = w->K / 32;
  int rb = moe::kGvLdsBudget / (KB * moe::kGvPitch);
  if (rb > moe::kGvMaxRB) rb = moe::kGvMaxRB;
  if (rb < 1) return MOE_ESHAPE;
  const int units = (act == MOE_ACT_SWIGLU_OAI) ? (w->N / 2 + 1) / 2 : (w->N + 3) / 4;
  int64_t slots = mpad_max / tile_m;
  if (slots > w->E) slots = w->E;
  // few live experts (decode): spread each expert's rows over many workgroups
  const int upw = (slots * units >= 8192) ? 2 : 1;
  const int64_t bx = (units + 4 * upw - 1) / (4 * upw);
  const size_t lds = (size_t)rb * KB * moe::kGvPitch;
  hipLaunchKernelGGL(moe::gemv_kernel, dim3((unsigned)bx, (unsigned)slots), dim3(moe::kGvThreads),
                     lds, stream, a, a_row, w->q, w->s, w->bias, counts, basep, w->E, w->N, w->K,
                     act, alpha, limit, out, rb, upw);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
