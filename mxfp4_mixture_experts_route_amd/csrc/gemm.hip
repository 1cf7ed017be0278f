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
//  * Weights are in the chunked layout (chunks of 4 MX blocks, all rows of a chunk together):
//    a wavefront's load of 16 rows x 4 blocks is one contiguous 1 KB run, and at any moment the
//    whole launch reads a compact window of the stack, which keeps HBM streaming at full rate
//    (the checkpoint's row-major layout scatters 64-byte pieces 1440 bytes apart).
//  * All global loads are buffer loads: each lane's offset is computed once, the chunk offset
//    rides in the scalar offset, and lanes with nothing to load point past the resource, which
//    returns zeros. The K loop therefore carries no per-lane guards and no 64-bit address math.
//  * MFMA v_mfma_f32_16x16x32_bf16 with the WEIGHTS as the 16-row A operand and the routed rows
//    (tokens) as the 16-column B operand: the token granule is 16, and each lane's output is 4
//    consecutive weight rows of one token (16-byte stores).
//  * MXFP4 -> bf16 happens in registers, never in LDS: an A fragment is 8 consecutive k of one
//    weight row, i.e. one dword of a 16-byte MX block, and v_cvt_scalef32_pk_bf16_fp4 turns it
//    into 4 VGPRs of bf16 with the block's e8m0 scale folded in (exact). A lane loads a whole
//    16-byte block (lanes 16g..16g+15 take block g of a 4-block chunk), and the 4 k-substeps of
//    the chunk take its 4 dwords; the activations are read from LDS in the same k order, and a
//    sum over k does not depend on that order beyond fp32 rounding.
//  * A ring of 4 chunks of weights (16 KB per wavefront) is in flight ahead of the MFMAs.
//  * Activation rows are gathered through a_row (row_tok) into LDS, 128 k per chunk, double
//    buffered; every B fragment read from LDS feeds 4 MFMAs (the wavefront's 4 weight tiles).
//  * Accumulators start at the bias of their weight row. Token tiles past the expert's count are
//    never computed; rows past the count are never stored. Experts with no rows exit at once.
//  * SwiGLU mode pairs gate tiles with the matching up tiles in the same wavefront, so the
//    epilogue is register-local and only bf16 h leaves the kernel.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kGmThreads = 256;          // 4 wavefronts
constexpr int kGmWT = 4;                 // weight tiles (16 rows each) per wavefront
constexpr int kGmTT = 8;                 // token tiles (16 rows each) per pass: 128 routed rows
constexpr int kGmChunkK = 128;           // k per chunk = 4 MX blocks
constexpr int kGmPF = 4;                 // weight chunks in flight per wavefront
constexpr int kGmPitch = kGmChunkK + 8;  // bf16 per LDS row (272 B: rows 4 banks apart)
constexpr int kGmBufElems = kGmTT * 16 * kGmPitch;
constexpr int kGmLdsBytes = 2 * kGmBufElems * 2;

// Everything one pass over up to 16*NTT routed rows of one expert needs.
struct GemmCtx {
  const int32_t* a_row;
  const float* bias;
  void* out;
  __amdgpu_buffer_rsrc_t rq, rs, ra;
  int e, N, K, C, klast, row0, p0, live, F;
  int tid, lr, lg;
  float alpha, limit;
  int tile_base[kGmWT];
  int rows_in[kGmWT];
  uint32_t wo[kGmWT], wol[kGmWT], so[kGmWT];
};

// One pass with NTT live token tiles (compile-time, so the MFMA loop is straight-line code and
// LDS reads can be scheduled ahead of the MFMAs that use them).
template <int ACT, int NTT>
__device__ __forceinline__ void gemm_pass(const GemmCtx& g, uint16_t* __restrict__ xs) {
  constexpr bool swiglu = (ACT == MOE_ACT_SWIGLU_OAI);
  const int C = g.C;
  const int lr = g.lr, lg = g.lg;

  // weight fetch of chunk c into a ring slot (zeros past K); c is uniform
  auto load_w = [&](int c, u32x4_t (&dq)[kGmWT], uint32_t (&dx)[kGmWT]) {
    if (c < C) {
      const uint32_t cq = (uint32_t)c * g.N * (kChunkBlocks * 16);
      const uint32_t cs = (uint32_t)c * kChunkBlocks;   // scale byte of block 4c + lg
      const bool last = (c == C - 1);
#pragma unroll
      for (int t = 0; t < kGmWT; ++t) {
        dq[t] = buf_load16(g.rq, last ? g.wol[t] : g.wo[t], cq);
        dx[t] = buf_load8(g.rs, g.so[t], cs);
      }
    } else {
#pragma unroll
      for (int t = 0; t < kGmWT; ++t) {
        dq[t] = u32x4_t{0u, 0u, 0u, 0u};
        dx[t] = 127u;
      }
    }
  };

  f32x4_t acc[kGmWT][NTT];
#pragma unroll
  for (int t = 0; t < kGmWT; ++t) {
    float b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * lg + i;
      b[i] = (g.bias && r < g.rows_in[t]) ? g.bias[(size_t)g.e * g.N + g.tile_base[t] + r] : 0.0f;
    }
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[t][tt] = f32x4_t{b[0], b[1], b[2], b[3]};
  }

  // activation staging: thread -> (row = tid/16 + 16*pass, 16-byte piece = tid%16)
  const int srow = g.tid >> 4, spiece = g.tid & 15;
  const bool piece_in_last = spiece * 8 < g.klast;
  uint32_t ao[NTT];
#pragma unroll
  for (int ps = 0; ps < NTT; ++ps) {
    const int m = ps * 16 + srow;
    uint32_t off = kOOB;
    if (m < g.live) {
      const int r = g.row0 + g.p0 + m;
      const uint32_t src = g.a_row ? (uint32_t)g.a_row[r] : (uint32_t)r;
      off = src * (uint32_t)g.K * 2 + spiece * 16;
    }
    ao[ps] = off;
  }
  uint4 stage[NTT];
  auto load_stage = [&](int c) {
    const uint32_t ck = (uint32_t)c * kGmChunkK * 2;
    const bool last = (c == C - 1);
#pragma unroll
    for (int ps = 0; ps < NTT; ++ps) {
      const u32x4_t v = buf_load16(g.ra, (last && !piece_in_last) ? kOOB : ao[ps], ck);
      stage[ps] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int ps = 0; ps < NTT; ++ps)
      *reinterpret_cast<uint4*>(xs + buf * kGmBufElems + (ps * 16 + srow) * kGmPitch +
                                spiece * 8) = stage[ps];
  };

  u32x4_t wq[kGmPF][kGmWT];
  uint32_t wx[kGmPF][kGmWT];

  load_stage(0);
  __syncthreads();  // previous pass is done with both LDS buffers
  store_stage(0);
  if (C > 1) load_stage(1);
#pragma unroll
  for (int pf = 0; pf < kGmPF; ++pf) load_w(pf, wq[pf], wx[pf]);

  for (int c0 = 0; c0 < C; c0 += kGmPF) {
#pragma unroll
    for (int pf = 0; pf < kGmPF; ++pf) {
      const int c = c0 + pf;
      if (c < C) {
        __syncthreads();  // chunk c is in LDS; buffer (c+1)&1 is free
        u32x4_t cq[kGmWT];
        float cs[kGmWT];
#pragma unroll
        for (int t = 0; t < kGmWT; ++t) {
          cq[t] = wq[pf][t];
          cs[t] = e8m0_scale_operand(wx[pf][t]);
        }
        load_w(c + kGmPF, wq[pf], wx[pf]);   // refill this ring slot (zeros past K)
        const uint16_t* xb = xs + (pf & 1) * kGmBufElems;   // c0 is even: c & 1 == pf & 1
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x8_t A[kGmWT];
#pragma unroll
          for (int t = 0; t < kGmWT; ++t) A[t] = dequant8(cq[t][i], cs[t]);
          bf16x8_t B[NTT];
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt)
            B[tt] = *reinterpret_cast<const bf16x8_t*>(xb + (tt * 16 + lr) * kGmPitch + lg * 32 +
                                                       i * 8);
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int t = 0; t < kGmWT; ++t)
              acc[t][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t], B[tt], acc[t][tt], 0, 0, 0);
        }
        if (c + 1 < C) {
          store_stage((pf + 1) & 1);
          if (c + 2 < C) load_stage(c + 2);
        }
      }
    }
  }

  // epilogue: lane holds rows 4*lg..4*lg+3 of each weight tile for token column lr
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int m = tt * 16 + lr;
    if (m >= g.live) continue;
    const size_t r = (size_t)(g.row0 + g.p0 + m);
    if (swiglu) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int j0 = g.tile_base[t] + 4 * lg;
        uint16_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          h[i] = (uint16_t)f32_to_bf16_bits(
              swiglu_oai(acc[t][tt][i], acc[t + 2][tt][i], g.alpha, g.limit));
        uint16_t* dst = reinterpret_cast<uint16_t*>(g.out) + r * g.F + j0;
        if (4 * lg + 4 <= g.rows_in[t] && (g.F & 3) == 0) {
          *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                                      (uint32_t)h[2] | ((uint32_t)h[3] << 16));
        } else {
          for (int i = 0; i < 4; ++i)
            if (4 * lg + i < g.rows_in[t]) dst[i] = h[i];
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < kGmWT; ++t) {
        float* dst = reinterpret_cast<float*>(g.out) + r * g.N + g.tile_base[t] + 4 * lg;
        if (4 * lg + 4 <= g.rows_in[t] && (g.N & 3) == 0) {
          *reinterpret_cast<f32x4_t*>(dst) = acc[t][tt];
        } else {
          for (int i = 0; i < 4; ++i)
            if (4 * lg + i < g.rows_in[t]) dst[i] = acc[t][tt][i];
        }
      }
    }
  }
}

template <int ACT>
__global__ void __launch_bounds__(kGmThreads)
gemm_kernel(const uint16_t* __restrict__ a, const int32_t* __restrict__ a_row, int a_rows,
            const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
            const float* __restrict__ bias, const int32_t* __restrict__ counts,
            const int32_t* __restrict__ basep, int E, int N, int K, float alpha, float limit,
            void* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  __shared__ int scratch[2];
  const int e = slot_expert(counts, E, (int)blockIdx.y, scratch);
  if (e < 0) return;
  constexpr bool swiglu = (ACT == MOE_ACT_SWIGLU_OAI);
  GemmCtx g;
  g.a_row = a_row;
  g.bias = bias;
  g.out = out;
  g.e = e;
  g.N = N;
  g.K = K;
  g.alpha = alpha;
  g.limit = limit;
  g.F = N >> 1;
  const int KB = K >> 5;
  g.C = (KB + kChunkBlocks - 1) / kChunkBlocks;             // chunks of 4 blocks
  const int wlast = KB - (g.C - 1) * kChunkBlocks;          // blocks in the last chunk
  g.klast = K - (g.C - 1) * kGmChunkK;                      // k in the last chunk
  g.tid = (int)threadIdx.x;
  const int lane = g.tid & 63, wave = g.tid >> 6;
  g.lr = lane & 15;
  g.lg = lane >> 4;
  g.row0 = basep[e];
  const int cnt = counts[e];

  // weight rows of the wavefront's 4 tiles (first row, rows that exist)
#pragma unroll
  for (int t = 0; t < kGmWT; ++t) {
    if (swiglu) {
      const int jb = (int)blockIdx.x * 128 + wave * 32 + (t & 1) * 16;
      g.tile_base[t] = (t < 2) ? jb : g.F + jb;
      g.rows_in[t] = min(16, g.F - jb);
    } else {
      g.tile_base[t] = (int)blockIdx.x * 256 + wave * 64 + t * 16;
      g.rows_in[t] = min(16, N - g.tile_base[t]);
    }
  }

  // buffer resources: this expert's nibbles and scales, and the activation rows
  const size_t ebase = (size_t)e * N * KB;   // first block of this expert (chunked layout)
  const int SP = scale_row_bytes(KB);        // scale row pitch (padding reads as 0)
  g.rq = make_rsrc(q + 16 * ebase, (uint32_t)N * KB * 16);
  g.rs = make_rsrc(s + (size_t)e * N * SP, (uint32_t)N * SP);
  g.ra = make_rsrc(a, (uint32_t)a_rows * K * 2);

  // per-lane offsets of the lane's block in a full chunk and in the (narrower) last chunk
#pragma unroll
  for (int t = 0; t < kGmWT; ++t) {
    const uint32_t n = (uint32_t)(g.tile_base[t] + g.lr);
    const bool ok = g.lr < g.rows_in[t];
    g.so[t] = ok ? n * SP + g.lg : kOOB;
    g.wo[t] = ok ? (n * kChunkBlocks + g.lg) * 16 : kOOB;
    g.wol[t] = (ok && g.lg < wlast) ? (n * wlast + g.lg) * 16 : kOOB;
  }

  for (int p0 = 0; p0 < cnt; p0 += kGmTT * 16) {
    g.p0 = p0;
    g.live = min(kGmTT * 16, cnt - p0);
    switch ((g.live + 15) >> 4) {
      case 1: gemm_pass<ACT, 1>(g, xs); break;
      case 2: gemm_pass<ACT, 2>(g, xs); break;
      case 3: gemm_pass<ACT, 3>(g, xs); break;
      case 4: gemm_pass<ACT, 4>(g, xs); break;
      case 5: gemm_pass<ACT, 5>(g, xs); break;
      case 6: gemm_pass<ACT, 6>(g, xs); break;
      case 7: gemm_pass<ACT, 7>(g, xs); break;
      default: gemm_pass<ACT, 8>(g, xs); break;
    }
  }
}

}  // namespace moe

int moe_launch_gemm(const uint16_t* a, const int32_t* a_row, int64_t a_rows, const mx4_experts* w,
                    const int32_t* counts, const int32_t* basep, int tile_m, int64_t mpad_max,
                    int act, float alpha, float limit, void* out, hipStream_t stream) {
  // buffer resources address at most 2 GB: one expert's weights and the activation matrix
  if ((int64_t)w->N * w->K / 2 >= (1LL << 31) || a_rows * w->K * 2 >= (1LL << 31))
    return MOE_ESHAPE;
  const int64_t bx = (act == MOE_ACT_SWIGLU_OAI) ? (w->N / 2 + 127) / 128 : (w->N + 255) / 256;
  int64_t slots = mpad_max / tile_m;
  if (slots > w->E) slots = w->E;
  static bool lds_attr_set = false;  // > 64 KB of dynamic LDS must be opted into once
  if (!lds_attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&moe::gemm_kernel<MOE_ACT_NONE>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            moe::kGmLdsBytes) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(&moe::gemm_kernel<MOE_ACT_SWIGLU_OAI>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            moe::kGmLdsBytes) != hipSuccess)
      return MOE_ELAUNCH;
    lds_attr_set = true;
  }
  if (act == MOE_ACT_SWIGLU_OAI)
    moe::launch(moe::gemm_kernel<MOE_ACT_SWIGLU_OAI>, dim3((unsigned)bx, (unsigned)slots),
                       dim3(moe::kGmThreads), moe::kGmLdsBytes, stream, a, a_row, (int)a_rows,
                       w->q, w->s, w->bias, counts, basep, w->E, w->N, w->K, alpha, limit, out);
  else
    moe::launch(moe::gemm_kernel<MOE_ACT_NONE>, dim3((unsigned)bx, (unsigned)slots),
                       dim3(moe::kGmThreads), moe::kGmLdsBytes, stream, a, a_row, (int)a_rows,
                       w->q, w->s, w->bias, counts, basep, w->E, w->N, w->K, alpha, limit, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
