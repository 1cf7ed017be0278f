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
// latency, so every weight load of a wavefront is in flight before it computes anything, and
// the per-byte instruction count is kept low so that compute trails the stream closely.
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
//  * The products run on v_mfma_f32_16x16x32_bf16: the 16 weight rows are the A operand and up to
//    16 routed rows of the expert (decode: usually one) are the B columns, so one MFMA does the
//    work of 16 dot2 instructions and the vector ALU only decodes. e2m1 nibbles are decoded by
//    v_cvt_scalef32_pk_bf16_fp4 (two codes to two bf16 with the block's e8m0 scale folded in;
//    exact). The 4 MFMA k-steps of a chunk take dword t of every lane's 16-byte block, and the
//    activations are read from LDS in the same k order (a sum over k does not depend on that
//    order beyond fp32 rounding).
//  * When every activation row fits (a_rows * K * 2 bytes <= 32 KB; decode) the workgroup copies
//    them all into LDS at kernel start with LDS-DMA buffer loads, before and independently of
//    the CSR; otherwise it stages the expert's rows per pass. The B fragments of chunk i + 2 are
//    read while chunk i is computed.
//  * Accumulators start at the bias of their row. Lane (q, c) ends with rows 4q..4q+3 of column
//    c; in SwiGLU mode rows 0-7 are gate rows and 8-15 the matching up rows, so one shuffle
//    pairs them and only bf16 h leaves the kernel.
#include "common.hpp"

namespace moe {

constexpr int kGvSeg = 24;        // chunks per K segment, all in flight at once (K <= 3072: one)
constexpr int kGvSegSplit = 12;   // the same when K is split over two wavefronts
constexpr int kGvCols = 16;       // routed rows per pass (MFMA B columns)
constexpr int kGvLdsBudget = 65536;
constexpr int kGvStageAll = 32768;  // all activation rows are staged up front up to this many bytes
constexpr int kGvMaxThreads = 256;
constexpr int kGvPF = 1;          // B fragments read this many chunks ahead

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
  if (stage_all) {
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, (uint32_t)a_rows * row_bytes);
    const int pieces = (int)(((uint32_t)a_rows * row_bytes + 1023) >> 10);
    for (int i = wave; i < pieces; i += (nthreads >> 6))
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(xs + (size_t)i * 1024), 16,
          (uint32_t)i * 1024 + (uint32_t)lane * 16, 0, 0, 0);
  }
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
  const int Cp = ((C + ksplit - 1) / ksplit + 3) & ~3;   // multiple of 4: whole scale dwords
  const int cb = part * Cp;
  const int ce = min(C, cb + Cp);
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
  const int SP = scale_row_bytes(KB);
  const int wlast = KB - (C - 1) * kChunkBlocks;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + 16 * (size_t)e * N * KB, (uint32_t)N * KB * 16);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s + (size_t)e * N * SP, (uint32_t)N * SP);
  const uint32_t wo = valid ? ((uint32_t)n * kChunkBlocks + lg) * 16 : kOOB;       // full chunk
  const uint32_t wol = (valid && lg < wlast) ? ((uint32_t)n * wlast + lg) * 16 : kOOB;  // last
  const uint32_t so = valid ? (uint32_t)n * SP : kOOB;

  // bias of the 4 accumulator rows this lane ends with (rows 4*lg .. 4*lg+3)
  float b4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bool ok;
    const int nn = row_of(4 * lg + i, ok);
    b4[i] = (ok && bias && part == 0) ? bias[(size_t)e * N + nn] : 0.0f;
  }

  // branch-free: a chunk past K or past this wavefront's part gets an out-of-range offset and
  // reads zeros
  auto load_chunk = [&](int c, u32x4_t& wq) {
    const uint32_t off = (c >= ce) ? kOOB : (c < C - 1 ? wo : wol);
    wq = buf_load16(rq, off, (uint32_t)c * N * (kChunkBlocks * 16));
  };
  // one K segment in K order: for every 4 chunks, their scale dwords, then their nibbles. The
  // scheduling barriers keep that issue order (the compiler would otherwise move the scale
  // loads last, and chunk 0 would then wait for the whole segment).
  u32x4_t wq[SEG];
  uint32_t sc[SEG];
  auto load_segment = [&](int c0) {
#pragma unroll
    for (int i = 0; i < SEG / 4; ++i) {
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
  load_segment(cb);

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

  // 5. one K segment for the B column of this lane (LDS blocks from xbase, or the zero block
  // for an empty column), accumulated into acc. Straight line (no branches, so each chunk waits
  // only for its own loads): blocks past K read zero weights and the zero activation block.
  auto run_segment = [&](int c0, const uint8_t* xbase, bool col_live, f32x4_t& acc0,
                         f32x4_t& acc1) {
    auto xaddr = [&](int i) {
      const int kb = (c0 + i) * kChunkBlocks + lg;
      return (col_live && kb < KB && c0 + i < ce) ? xbase + (size_t)kb * 64 : xzero;
    };
    bf16x8_t xv[kGvPF + 1][4];
#pragma unroll
    for (int p = 0; p < kGvPF; ++p)
#pragma unroll
      for (int t = 0; t < 4; ++t) xv[p][t] = *reinterpret_cast<const bf16x8_t*>(xaddr(p) + 16 * t);
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      // chunks past this wavefront's part read zero weights; their scale byte may belong to the
      // next part (and be the NaN byte), so it is replaced by 0
      const uint32_t eb = (c0 + i < ce) ? __builtin_amdgcn_ubfe(sc[i], 8 * lg, 8) : 0u;
      const float scl = e8m0_scale_operand(eb);
      if (i + kGvPF < SEG) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          xv[(i + kGvPF) % (kGvPF + 1)][t] =
              *reinterpret_cast<const bf16x8_t*>(xaddr(i + kGvPF) + 16 * t);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4_t& acc = (t & 1) ? acc1 : acc0;   // two chains: back-to-back MFMAs stay independent
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(wq[i][t], scl),
                                                      xv[i % (kGvPF + 1)][t], acc, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the B reads kGvPF chunks ahead of their use
    }
  };

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
      if (!one_seg && (c0 > cb || p0 > 0)) load_segment(c0);
      run_segment(c0, xbase, col_live, acc, acc1);
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
  hipLaunchKernelGGL((moe::gemv_kernel<ACT, SEG>), grid, block, lds, stream, a, a_row, (int)a_rows,
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
  // K over two wavefronts when it takes more than one short segment: twice the wavefronts,
  // each with half the loads in flight, keep the decode closer behind the weight stream
  const int ksplit = C > moe::kGvSegSplit ? 2 : 1;
  // Wavefronts per workgroup: as many as keep >= ~2.5 workgroups per CU (256 CUs), so that the
  // uneven last round of workgroups costs little; more wavefronts share one activation staging.
  const int64_t total_waves = (int64_t)units * slots * ksplit;
  int waves = 4;
  while (waves > ksplit && total_waves / waves < 640) waves >>= 1;
  const int threads = 64 * waves;
  const size_t all_bytes = ((size_t)a_rows * row_bytes + 1023) & ~(size_t)1023;
  const int stage_all = all_bytes <= (size_t)moe::kGvStageAll ? 1 : 0;
  int rb = (int)((moe::kGvLdsBudget - 64) / row_bytes);   // rows + the zero block
  if (rb > moe::kGvCols) rb = moe::kGvCols;
  if (rb < 1) return MOE_ESHAPE;
  const size_t lds = (stage_all ? all_bytes : (size_t)rb * row_bytes) + 64 +
                     (ksplit > 1 ? (size_t)threads * 16 : 0);
  const int64_t bx = (units + waves / ksplit - 1) / (waves / ksplit);
  const dim3 grid((unsigned)bx, (unsigned)slots), block((unsigned)threads);
  if (act == MOE_ACT_SWIGLU_OAI) {
    if (ksplit > 1)
      launch_gemv<MOE_ACT_SWIGLU_OAI, moe::kGvSegSplit>(grid, block, lds, stream, a, a_row, a_rows, w,
                                                         counts, basep, alpha, limit, out, rb,
                                                         stage_all, ksplit);
    else
      launch_gemv<MOE_ACT_SWIGLU_OAI, moe::kGvSeg>(grid, block, lds, stream, a, a_row, a_rows, w,
                                                    counts, basep, alpha, limit, out, rb,
                                                    stage_all, ksplit);
  } else {
    if (ksplit > 1)
      launch_gemv<MOE_ACT_NONE, moe::kGvSegSplit>(grid, block, lds, stream, a, a_row, a_rows, w,
                                                   counts, basep, alpha, limit, out, rb, stage_all,
                                                   ksplit);
    else
      launch_gemv<MOE_ACT_NONE, moe::kGvSeg>(grid, block, lds, stream, a, a_row, a_rows, w, counts,
                                              basep, alpha, limit, out, rb, stage_all, ksplit);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
