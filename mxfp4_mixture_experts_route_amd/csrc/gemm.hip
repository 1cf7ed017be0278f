// mx4_moe_gemm: routed-expert MXFP4 projection for prefill, on bf16 MFMA with fp32 accumulation.
//
// Sources: PR #3579 "dasLLAMA gpt-oss arc", Metal fusion-lane commit (the grouped expert matmul
// over the buckets starts its accumulator tiles from the expert's bias row instead of running a
// separate bias pass; the SwiGLU-OAI epilogue skips ghost rows past the last padded bucket end);
// PR #3558 "dasLLAMA: dig the last two board reds green", section "gpt-oss: mx4 kernels to the
// lab-winning shape" (the matmul's weight stage: 16-byte block loads, e2m1 table decode, e8m0
// applied arithmetically).
//
// gfx950 mapping. One workgroup (4 wavefronts) owns one expert and one slice of weight rows and
// runs over all of that expert's routed rows, so every weight byte is fetched from HBM once.
//  * MFMA v_mfma_f32_16x16x32_bf16 with the WEIGHTS as the 16-row A operand and the routed rows
//    (tokens) as the 16-column B operand: the token granule is 16, and each lane's output is 4
//    consecutive weight rows of one token (16-byte stores).
//  * MXFP4 -> bf16 happens in registers, never in LDS: an A fragment is 8 consecutive k of one
//    weight row, i.e. one dword of a 16-byte MX block, and v_cvt_scalef32_pk_bf16_fp4 turns it
//    into 4 VGPRs of bf16 with the block's e8m0 scale folded in (exact). A lane loads a whole
//    16-byte block (lanes 16g..16g+15 take block g of a 4-block chunk), and the 4 k-substeps of
//    the chunk take its 4 dwords; the activations are read from LDS in the same k order, and a
//    sum over k does not depend on that order beyond fp32 rounding.
//  * Activation rows are gathered through a_row (row_tok) into LDS, 128 k per chunk, double
//    buffered; every B fragment read from LDS feeds 4 MFMAs (the wavefront's 4 weight tiles).
//  * Accumulators start at the bias of their weight row. Token tiles past the expert's count are
//    never computed; rows past the count are never stored. Experts with no rows exit at once.
//  * SwiGLU mode pairs gate tiles with the matching up tiles in the same wavefront, so the
//    epilogue is register-local and only bf16 h leaves the kernel.
#include "common.hpp"

namespace moe {

constexpr int kGmThreads = 256;          // 4 wavefronts
constexpr int kGmWT = 4;                 // weight tiles (16 rows each) per wavefront
constexpr int kGmTT = 8;                 // token tiles (16 rows each) per pass: 128 routed rows
constexpr int kGmChunkK = 128;           // k per chunk = 4 MX blocks
constexpr int kGmPitch = kGmChunkK + 8;  // bf16 per LDS row (272 B: rows 4 banks apart)
constexpr int kGmBufElems = kGmTT * 16 * kGmPitch;
constexpr int kGmLdsBytes = 2 * kGmBufElems * 2;

__device__ __forceinline__ bf16x8_t dequant8(uint32_t w8, float scale) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w8, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w8, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w8, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w8, scale, 3);
  return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__global__ void __launch_bounds__(kGmThreads)
gemm_kernel(const uint16_t* __restrict__ a, const int32_t* __restrict__ a_row,
            const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
            const float* __restrict__ bias, const int32_t* __restrict__ counts,
            const int32_t* __restrict__ basep, int E, int N, int K, int act, float alpha,
            float limit, void* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  __shared__ int scratch[2];
  const int e = slot_expert(counts, E, (int)blockIdx.y, scratch);
  if (e < 0) return;
  const int cnt = counts[e];
  const int row0 = basep[e];
  const int KB = K >> 5;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const bool swiglu = (act == MOE_ACT_SWIGLU_OAI);
  const int F = N >> 1;
  const size_t row_bytes = (size_t)K >> 1;

  // weight rows: A-operand row of this lane in each tile, and the first row of each tile
  int tile_base[kGmWT];
  int rows_in[kGmWT];  // rows of the tile that exist (N or F tail)
#pragma unroll
  for (int t = 0; t < kGmWT; ++t) {
    if (swiglu) {
      const int jb = (int)blockIdx.x * 128 + wave * 32 + (t & 1) * 16;
      tile_base[t] = (t < 2) ? jb : F + jb;
      rows_in[t] = min(16, F - jb);
    } else {
      tile_base[t] = (int)blockIdx.x * 256 + wave * 64 + t * 16;
      rows_in[t] = min(16, N - tile_base[t]);
    }
  }
  const uint8_t* qe = q + (size_t)e * N * row_bytes;
  const uint8_t* se = s + (size_t)e * N * KB;
  const int nchunks = (K + kGmChunkK - 1) / kGmChunkK;

  for (int p0 = 0; p0 < cnt; p0 += kGmTT * 16) {
    const int live = min(kGmTT * 16, cnt - p0);
    const int ntt = (live + 15) >> 4;

    f32x4_t acc[kGmWT][kGmTT];
#pragma unroll
    for (int t = 0; t < kGmWT; ++t) {
      float b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * lg + i;
        b[i] = (bias && r < rows_in[t]) ? bias[(size_t)e * N + tile_base[t] + r] : 0.0f;
      }
#pragma unroll
      for (int tt = 0; tt < kGmTT; ++tt) acc[t][tt] = f32x4_t{b[0], b[1], b[2], b[3]};
    }

    // activation staging: thread -> (row = tid/16 + 16*pass, 16-byte piece = tid%16)
    const int srow = tid >> 4, spiece = tid & 15;
    int64_t src_row[kGmTT];
#pragma unroll
    for (int ps = 0; ps < kGmTT; ++ps) {
      const int m = ps * 16 + srow;
      if (m < live) {
        const int r = row0 + p0 + m;
        src_row[ps] = a_row ? (int64_t)a_row[r] : (int64_t)r;
      } else {
        src_row[ps] = -1;
      }
    }
    uint4 stage[kGmTT];
    auto load_stage = [&](int c) {
#pragma unroll
      for (int ps = 0; ps < kGmTT; ++ps) {
        const int k = c * kGmChunkK + spiece * 8;
        if (ps < ntt && src_row[ps] >= 0 && k < K)
          stage[ps] = *reinterpret_cast<const uint4*>(a + src_row[ps] * K + k);
        else
          stage[ps] = make_uint4(0u, 0u, 0u, 0u);
      }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
      for (int ps = 0; ps < kGmTT; ++ps)
        if (ps < ntt)
          *reinterpret_cast<uint4*>(xs + buf * kGmBufElems + (ps * 16 + srow) * kGmPitch +
                                    spiece * 8) = stage[ps];
    };
    // weight fetch: lane takes block (chunk*4 + lg) of its row in each tile
    u32x4_t wq[kGmWT];
    uint32_t wx[kGmWT];
    auto load_w = [&](int c) {
      const int kb = c * 4 + lg;
#pragma unroll
      for (int t = 0; t < kGmWT; ++t) {
        if (lr < rows_in[t] && kb < KB) {
          const size_t n = (size_t)(tile_base[t] + lr);
          wq[t] = *reinterpret_cast<const u32x4_t*>(qe + n * row_bytes + (size_t)kb * 16);
          wx[t] = se[n * KB + kb];
        } else {
          wq[t] = u32x4_t{0u, 0u, 0u, 0u};
          wx[t] = 127u;
        }
      }
    };

    load_stage(0);
    __syncthreads();  // previous pass is done with both LDS buffers
    store_stage(0);
    if (nchunks > 1) load_stage(1);
    load_w(0);

    for (int c = 0; c < nchunks; ++c) {
      __syncthreads();  // chunk c is in LDS; buffer (c+1)&1 is free
      const u32x4_t cq[kGmWT] = {wq[0], wq[1], wq[2], wq[3]};
      float cs[kGmWT];
#pragma unroll
      for (int t = 0; t < kGmWT; ++t) cs[t] = e8m0_to_f32(wx[t]);
      if (c + 1 < nchunks) load_w(c + 1);
      const uint16_t* xb = xs + (c & 1) * kGmBufElems;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8_t A[kGmWT];
#pragma unroll
        for (int t = 0; t < kGmWT; ++t) A[t] = dequant8(cq[t][i], cs[t]);
#pragma unroll
        for (int tt = 0; tt < kGmTT; ++tt) {
          if (tt < ntt) {
            const bf16x8_t B = *reinterpret_cast<const bf16x8_t*>(
                xb + (tt * 16 + lr) * kGmPitch + lg * 32 + i * 8);
#pragma unroll
            for (int t = 0; t < kGmWT; ++t)
              acc[t][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t], B, acc[t][tt], 0, 0, 0);
          }
        }
      }
      if (c + 1 < nchunks) {
        store_stage((c + 1) & 1);
        if (c + 2 < nchunks) load_stage(c + 2);
      }
    }

    // epilogue: lane holds rows 4*lg..4*lg+3 of each weight tile for token column lr
#pragma unroll
    for (int tt = 0; tt < kGmTT; ++tt) {
      if (tt >= ntt) continue;
      const int m = tt * 16 + lr;
      if (m >= live) continue;
      const size_t r = (size_t)(row0 + p0 + m);
      if (swiglu) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int j0 = tile_base[t] + 4 * lg;
          uint16_t h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            h[i] = (uint16_t)f32_to_bf16_bits(swiglu_oai(acc[t][tt][i], acc[t + 2][tt][i], alpha, limit));
          uint16_t* dst = reinterpret_cast<uint16_t*>(out) + r * F + j0;
          if (4 * lg + 4 <= rows_in[t] && (F & 3) == 0) {
            *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                                        (uint32_t)h[2] | ((uint32_t)h[3] << 16));
          } else {
            for (int i = 0; i < 4; ++i)
              if (4 * lg + i < rows_in[t]) dst[i] = h[i];
          }
        }
      } else {
#pragma unroll
        for (int t = 0; t < kGmWT; ++t) {
          float* dst = reinterpret_cast<float*>(out) + r * N + tile_base[t] + 4 * lg;
          if (4 * lg + 4 <= rows_in[t] && (N & 3) == 0) {
            *reinterpret_cast<f32x4_t*>(dst) = acc[t][tt];
          } else {
            for (int i = 0; i < 4; ++i)
              if (4 * lg + i < rows_in[t]) dst[i] = acc[t][tt][i];
          }
        }
      }
    }
  }
}

}  // namespace moe

int moe_launch_gemm(const uint16_t* a, const int32_t* a_row, const mx4_experts* w,
                    const int32_t* counts, const int32_t* basep, int tile_m, int64_t mpad_max,
                    int act, float alpha, float limit, void* out, hipStream_t stream) {
  const int64_t bx = (act == MOE_ACT_SWIGLU_OAI) ? (w->N / 2 + 127) / 128 : (w->N + 255) / 256;
  int64_t slots = mpad_max / tile_m;
  if (slots > w->E) slots = w->E;
  static bool lds_attr_set = false;  // > 64 KB of dynamic LDS must be opted into once
  if (!lds_attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&moe::gemm_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            moe::kGmLdsBytes) != hipSuccess)
      return MOE_ELAUNCH;
    lds_attr_set = true;
  }
  hipLaunchKernelGGL(moe::gemm_kernel, dim3((unsigned)bx, (unsigned)slots), dim3(moe::kGmThreads),
                     moe::kGmLdsBytes, stream, a, a_row, w->q, w->s, w->bias, counts, basep, w->E,
                     w->N, w->K, act, alpha, limit, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
