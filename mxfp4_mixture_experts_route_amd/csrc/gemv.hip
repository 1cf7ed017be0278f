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
// gfx950 mapping: the wavefront engine of gemv_core.hpp (weights streamed in the chunked layout,
// a whole K segment in flight per wavefront, bf16 MFMA with the routed rows as B columns). Per
// workgroup and expert:
//  * Each wavefront finds its expert by itself (one load of counts[], a ballot).
//  * When every activation row fits (a_rows * K * 2 bytes <= 32 KB; decode) the workgroup copies
//    them all into LDS at kernel start with LDS-DMA buffer loads, before and independently of
//    the CSR; otherwise it stages the expert's rows per pass of up to 16.
//  * With K longer than one short segment, K is split over wavefront pairs and the partial sums
//    meet in LDS.
//  * Accumulators start at the bias of their row. In SwiGLU mode rows 0-7 of a wavefront are
//    gate rows and 8-15 the matching up rows, so one shuffle pairs them and only bf16 h leaves
//    the kernel; rows that are not live are never written.
#include "gemv_core.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kGvCols = 16;       // routed rows per pass (MFMA B columns)
constexpr int kGvLdsBudget = 65536;
constexpr int kGvStageAll = 32768;  // all activation rows are staged up front up to this many bytes
constexpr int kGvMaxThreads = 256;

template <int ACT, int SEG>
__global__ void __launch_bounds__(kGvMaxThreads)
gemv_kernel(const uint16_t* __restrict__ a, const int32_t* __restrict__ a_row, int a_rows,
            const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
            const float* __restrict__ bias, const int32_t* __restrict__ counts,
            const int32_t* __restrict__ basep, int E, int N, int K, float alpha, float limit,
            void* __restrict__ out, int rb, int stage_all, int ksplit) {
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
  // 1. counts for the expert lookup, then (when they all fit) every activation row, copied
  // global -> LDS by the load unit itself (LDS-DMA buffer loads: no registers, and the copy is
  // byte for byte, so activation row r sits at xs + r * K * 2); wavefront w copies the 1 KB
  // pieces w, w + W, ...; bytes past the rows read as zeros
  const int c64 = (lane < E) ? counts[lane] : 0;
  const uint32_t row_bytes = (uint32_t)K * 2;
  if (stage_all) lds_dma_copy(a, (uint32_t)a_rows * row_bytes, xs, wave, nthreads >> 6);
  __builtin_amdgcn_sched_barrier(0);

  // 2. expert of this workgroup's slot (each wavefront on its own)
  const int e = wave_slot_expert(counts, E, (int)blockIdx.y, c64);
  if (e < 0) {  // uniform over the workgroup: fewer live experts than slots
    __builtin_amdgcn_s_waitcnt(0);   // no LDS-DMA write may outlive the workgroup's LDS
    return;
  }

  // 3. this wavefront's 16 weight rows (local row rho = 0..15 is weight row row_of(rho)) and its
  // part of K: with ksplit > 1, consecutive wavefronts take consecutive ranges of Cp chunks of
  // the same rows and are summed at the end
  const int part = wave % ksplit;
  const int unit = (int)blockIdx.x * ((nthreads >> 6) / ksplit) + wave / ksplit;
  int cb, ce, Cp;
  k_part_range(C, part, ksplit, cb, ce, Cp);
  auto row_of = [&](int rho, bool& ok) {
    if (swiglu) {
      const int jj = unit * 8 + (rho & 7);
      ok = jj < F;
      return rho < 8 ? jj : F + jj;
    }
    const int nn = unit * 16 + rho;
    ok = nn < N;
    return nn;
  };
  bool valid;
  const int n = row_of(lr, valid);   // A operand row of this lane
  Mx4Wave<SEG> ws;
  ws.init(q, s, e, n, valid, N, K, ce);

  // bias of the 4 accumulator rows this lane ends with (rows 4*lg .. 4*lg+3)
  float b4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bool ok;
    const int nn = row_of(4 * lg + i, ok);
    b4[i] = (ok && bias && part == 0) ? bias[(size_t)e * N + nn] : 0.0f;
  }

  ws.load_segment(cb);

  const int cnt = counts[e];
  const int row0 = basep[e];

  // 4. the all-zero block after the staged rows (read by empty columns and blocks past K)
  const size_t zero_off = stage_all ? (((size_t)a_rows * row_bytes + 1023) & ~(size_t)1023)
                                    : (size_t)rb * row_bytes;
  if (tid < 4) *reinterpret_cast<uint4*>(xs + zero_off + tid * 16) = make_uint4(0u, 0u, 0u, 0u);
  const uint8_t* xzero = xs + zero_off;
  const size_t red_off = zero_off + 64;   // K-part partial sums: one f32x4 per lane
  // the LDS-DMA copies were issued before the bias and the segment's weight loads, and vector
  // loads complete in order: once at most those are outstanding, the copies have landed (the
  // barrier at the start of the first pass then publishes them to the whole workgroup)
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(SEG + SEG / 4));

  // 6. the expert's rows in passes of up to 16 (one per B column); with K in one segment
  // (K <= 3072) the weights stay in registers for all passes, otherwise every pass streams the
  // segments again
  const bool one_seg = Cp <= SEG;
  const int pass_rows = stage_all ? kGvCols : rb;
  for (int p0 = 0; p0 < cnt; p0 += pass_rows) {
    const int nr = min(pass_rows, cnt - p0);
    if (!stage_all) {
      __syncthreads();  // the previous pass is done with xs
      for (int p = tid; p < nr * KB * 4; p += nthreads) {
        const int rr = p / (KB * 4);
        const int rem = p - rr * KB * 4;
        const int r = row0 + p0 + rr;
        const int64_t src = a_row ? (int64_t)a_row[r] : (int64_t)r;
        const uint4 v = *reinterpret_cast<const uint4*>(a + src * K + rem * 8);
        *reinterpret_cast<uint4*>(xs + (size_t)rr * row_bytes + (size_t)rem * 16) = v;
      }
    }
    __syncthreads();
    // LDS row of this lane's column lr (routed row row0 + p0 + lr): read with uniform loads
    int xr = 0;
    if (stage_all) {
      for (int c = 0; c < nr; ++c) {
        const int r = row0 + p0 + c;
        const int v = a_row ? a_row[r] : r;
        xr = (lr == c) ? v : xr;
      }
    } else {
      xr = lr;
    }
    const bool col_live = lr < nr;
    const uint8_t* xbase = xs + (size_t)xr * row_bytes;
    f32x4_t acc = {b4[0], b4[1], b4[2], b4[3]};   // bias-seeded accumulator
    f32x4_t acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c0 = cb; c0 < ce; c0 += SEG) {
      if (!one_seg && (c0 > cb || p0 > 0)) ws.load_segment(c0);
      ws.run_segment(c0, KB, xbase, xzero, col_live, acc, acc1);
    }
    acc += acc1;
    if (ksplit > 1) {
      // the parts of K meet in LDS; part 0 adds them in part order and does the epilogue
      f32x4_t* red = reinterpret_cast<f32x4_t*>(xs + red_off);
      if (part > 0) red[wave * 64 + lane] = acc;
      __syncthreads();
      if (part > 0) continue;
      for (int pp = 1; pp < ksplit; ++pp) acc += red[(wave + pp) * 64 + lane];
    }
    // lane (lg, lr) holds rows 4*lg + i of column lr
    const size_t r = (size_t)(row0 + p0 + lr);
    if (swiglu) {
      float up[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) up[i] = __shfl_xor(acc[i], 32);
      if (lg < 2 && col_live) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int jj = unit * 8 + 4 * lg + i;
          if (jj < F) {
            const float h = swiglu_oai(acc[i], up[i], alpha, limit);
            reinterpret_cast<uint16_t*>(out)[r * F + jj] = (uint16_t)f32_to_bf16_bits(h);
          }
        }
      }
    } else if (col_live) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nn = unit * 16 + 4 * lg + i;
        if (nn < N) reinterpret_cast<float*>(out)[r * N + nn] = acc[i];
      }
    }
  }
}

}  // namespace moe

// Host launcher shared with the C ABI entry point (argument checks are done by the caller).
template <int ACT, int SEG>
static void launch_gemv(dim3 grid, dim3 block, size_t lds, hipStream_t stream, const uint16_t* a,
                        const int32_t* a_row, int64_t a_rows, const mx4_experts* w,
                        const int32_t* counts, const int32_t* basep, float alpha, float limit,
                        void* out, int rb, int stage_all, int ksplit) {
  moe::launch((moe::gemv_kernel<ACT, SEG>), grid, block, lds, stream, a, a_row, (int)a_rows,
                     w->q, w->s, w->bias, counts, basep, w->E, w->N, w->K, alpha, limit, out, rb,
                     stage_all, ksplit);
}

int moe_launch_gemv(const uint16_t* a, const int32_t* a_row, int64_t a_rows, const mx4_experts* w,
                    const int32_t* counts, const int32_t* basep, int tile_m, int64_t mpad_max,
                    int act, float alpha, float limit, void* out, hipStream_t stream) {
  const size_t row_bytes = (size_t)w->K * 2;
  const int C = (w->K / 32 + moe::kChunkBlocks - 1) / moe::kChunkBlocks;
  const int units = (act == MOE_ACT_SWIGLU_OAI) ? (w->N / 2 + 7) / 8 : (w->N + 15) / 16;
  int64_t slots = mpad_max / tile_m;
  if (slots > w->E) slots = w->E;
  // K over up to 4 wavefronts (12 chunks each): shorter wavefronts keep the decode close behind
  // the weight stream. Row groups per workgroup: as many as keep >= ~2.5 workgroups per CU (256
  // CUs); more wavefronts share one activation staging.
  const int ksplit = moe::gv_ksplit(C);
  const int64_t total_waves = (int64_t)units * slots * ksplit;
  int upw = moe::kGvMaxThreads / 64 / ksplit;   // row groups per workgroup
  while (upw > 1 && total_waves / (upw * ksplit) < 640) upw >>= 1;
  const int waves = upw * ksplit;
  const int threads = 64 * waves;
  const size_t all_bytes = ((size_t)a_rows * row_bytes + 1023) & ~(size_t)1023;
  const int stage_all = all_bytes <= (size_t)moe::kGvStageAll ? 1 : 0;
  int rb = (int)((moe::kGvLdsBudget - 64 - (size_t)threads * 16) / row_bytes);
  if (rb > moe::kGvCols) rb = moe::kGvCols;
  if (rb < 1) return MOE_ESHAPE;
  const size_t lds = (stage_all ? all_bytes : (size_t)rb * row_bytes) + 64 +
                     (ksplit > 1 ? (size_t)threads * 16 : 0);
  const int64_t bx = (units + upw - 1) / upw;
  const dim3 grid((unsigned)bx, (unsigned)slots), block((unsigned)threads);
  if (act == MOE_ACT_SWIGLU_OAI)
    launch_gemv<MOE_ACT_SWIGLU_OAI, moe::kGvSeg>(grid, block, lds, stream, a, a_row, a_rows, w,
                                                  counts, basep, alpha, limit, out, rb, stage_all,
                                                  ksplit);
  else
    launch_gemv<MOE_ACT_NONE, moe::kGvSeg>(grid, block, lds, stream, a, a_row, a_rows, w, counts,
                                            basep, alpha, limit, out, rb, stage_all, ksplit);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
