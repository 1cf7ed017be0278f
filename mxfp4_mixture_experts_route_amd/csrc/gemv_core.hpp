// Wavefront engine of the decode-size MXFP4 projections (mx4_moe_gemv and the fused decode
// layer): one wavefront streams 16 weight rows of one expert over a range of K and multiplies
// them with up to 16 activation rows staged in LDS, on bf16 MFMA.
//
// Sources: PR #3558 "dasLLAMA: dig the last two board reds green", section "gpt-oss: mx4 kernels
// to the lab-winning shape" and its ladder table (routed-expert GEMV at gpt-oss shape: every
// weight byte loaded once; e2m1 decoded through a 16-entry table; the e8m0 exponent applied
// arithmetically rather than through a dependent table load).
//
// gfx950 mapping (HBM-bound; at tens of MB per launch the time goes to memory latency, so every
// weight load of a wavefront is in flight before it computes anything, and the per-byte
// instruction count stays low so that compute trails the stream closely):
//  * Weights are in the chunked layout (chunks of 4 MX blocks, all rows of a chunk together).
//    Lane (r = lane%16, g = lane/16) takes block g of every chunk of row r, so each load
//    instruction of the wavefront reads one contiguous 1 KB run.
//  * A segment of SEG = 12 chunks is loaded at once, in K order: for every 4 chunks their scale
//    dword group (one dwordx4: a lane's scale for chunk c is byte g of dword c of its 16-byte
//    padded scale row), then their nibbles. Loads complete in issue order, so chunk i is computed
//    as soon as its own bytes arrive. All loads are buffer loads with offsets computed once;
//    lanes or chunks with nothing to load point past the resource and read zeros.
//  * v_mfma_f32_16x16x32_bf16: the 16 weight rows are the A operand, the activation rows the B
//    columns (one MFMA does the work of 16 dot2 instructions, so the vector ALU only decodes).
//    e2m1 -> bf16 by v_cvt_scalef32_pk_bf16_fp4 with the block's e8m0 scale folded in (exact).
//    The 4 MFMA k-steps of a chunk take dword t of every lane's 16-byte block; the activations
//    are read from LDS in the same k order (a sum over k does not depend on that order beyond
//    fp32 rounding). B fragments are read kGvPF chunks ahead; two accumulator chains alternate.
//  * Lane (q, c) ends with rows 4q..4q+3 of B column c.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kGvSeg = 12;        // chunks per K segment and wavefront, all in flight at once
constexpr int kGvMaxSplit = 4;    // K is split over up to this many wavefronts of the same rows

// Wavefronts that share one set of 16 rows: one per 12 chunks of K, at most 4 (longer K runs
// several segments per wavefront). (Measured at gpt-oss K = 23 chunks: 2 wavefronts of 12 beat
// 3 of 8, whose smaller workgroups stage the activations twice as often.)
__host__ __device__ constexpr int gv_ksplit(int C) {
  return C <= kGvSeg ? 1 : (C + kGvSeg - 1) / kGvSeg > kGvMaxSplit ? kGvMaxSplit
                                                                   : (C + kGvSeg - 1) / kGvSeg;
}
constexpr int kGvPF = 1;          // B fragments read this many chunks ahead

// Expert of a slot: the slot-th expert with a non-zero count, or -1. c64 is this lane's
// counts[lane] (0 past E), loaded by the caller before anything else; experts past 64 are
// scanned 64 at a time. No LDS, no barrier.
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

// Issue LDS-DMA copies of `bytes` bytes at src into LDS at dst (both 16-byte aligned), in 1 KB
// pieces: wavefront `wave` of `waves` copies pieces wave, wave + waves, ...; bytes past `bytes`
// (up to the next KB) are written as zeros. Completion is tracked by the vector-memory counter.
__device__ __forceinline__ void lds_dma_copy(const void* src, uint32_t bytes, uint8_t* dst,
                                             int wave, int waves) {
  const int lane = (int)(threadIdx.x & 63);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src, bytes);
  const int pieces = (int)((bytes + 1023) >> 10);
  for (int i = wave; i < pieces; i += waves)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(dst + (size_t)i * 1024), 16,
        (uint32_t)i * 1024 + (uint32_t)lane * 16, 0, 0, 0);
}

template <int SEG>
struct Mx4Wave {
  __amdgpu_buffer_rsrc_t rq, rs;
  uint32_t wo, wol, so;
  int C, ce, G, N, lg;
  u32x4_t wq[SEG];
  uint32_t sc[SEG];

  // Rows of expert e (the same on every lane of the wavefront): this lane streams row n (if
  // valid) of an [E][N][K] chunked stack, over chunks [.., ce_) of the C chunks of K.
  __device__ __forceinline__ void init(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                       int e, int n, bool valid, int N_, int K, int ce_) {
    // e (and the K range, from the wavefront index) arrive in vector registers; read as scalars,
    // the buffer resources and scalar offsets below are scalars too (one in vector registers
    // makes the compiler wrap every load of the segment in a loop over the lanes' values)
    e = __builtin_amdgcn_readfirstlane(e);
    N_ = __builtin_amdgcn_readfirstlane(N_);
    K = __builtin_amdgcn_readfirstlane(K);
    ce_ = __builtin_amdgcn_readfirstlane(ce_);
    const int lane = (int)(threadIdx.x & 63);
    lg = lane >> 4;
    N = N_;
    const int KB = K >> 5;
    C = (KB + kChunkBlocks - 1) / kChunkBlocks;
    ce = ce_;
    G = scale_row_bytes(KB) / 16;
    const int wlast = KB - (C - 1) * kChunkBlocks;
    rq = make_rsrc(q + 16 * (size_t)e * N * KB, (uint32_t)N * KB * 16);
    rs = make_rsrc(s + (size_t)e * N * G * 16, (uint32_t)N * G * 16);
    wo = valid ? ((uint32_t)n * kChunkBlocks + lg) * 16 : kOOB;                // full chunk
    wol = (valid && lg < wlast) ? ((uint32_t)n * wlast + lg) * 16 : kOOB;      // last chunk
    so = valid ? (uint32_t)n * 16 : kOOB;   // the row's 16 bytes in a scale group
  }

  // Chunks [c0, c0 + SEG): scales and nibbles, in K order. A chunk past K or past ce reads
  // zeros (branch-free); a scale group past the last one reads zeros (it would otherwise read
  // another expert's scales, where a NaN byte would poison 0 * scale). The
  // scheduling barriers keep the issue order (the compiler would move the scale loads last).
  __device__ __forceinline__ void load_segment(int c0) {
    c0 = __builtin_amdgcn_readfirstlane(c0);   // uniform: the chunk offsets ride in soffset
#pragma unroll
    for (int i = 0; i < SEG / 4; ++i) {
      const int gi = (c0 + 4 * i) / 4;   // c0 is a multiple of 4: whole groups
      const u32x4_t v = buf_load16_nt(rs, gi < G ? so : kOOB, (uint32_t)gi * N * 16);
      sc[4 * i + 0] = v[0];
      sc[4 * i + 1] = v[1];
      sc[4 * i + 2] = v[2];
      sc[4 * i + 3] = v[3];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = c0 + 4 * i + k;
        const uint32_t off = (c >= ce) ? kOOB : (c < C - 1 ? wo : wol);
        wq[4 * i + k] = buf_load16_nt(rq, off, (uint32_t)c * N * (kChunkBlocks * 16));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Multiply the loaded segment starting at chunk c0 with the B column of this lane (activation
  // blocks from xbase, or the zero block xzero when the column is empty), into acc0/acc1.
  // Straight line (no branches, so each chunk waits only for its own loads): chunks past K or
  // past ce read zero weights and the zero activation block; their scale byte may belong to
  // another range (and be the NaN byte), so it is replaced by 0.
  __device__ __forceinline__ void run_segment(int c0, int KB, const uint8_t* xbase,
                                              const uint8_t* xzero, bool col_live, f32x4_t& acc0,
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
  }
};

// Chunk range [cb, ce) of K part `part` of `ksplit`: parts take Cp chunks each, Cp a multiple of
// 4 (whole scale dword groups). gpt-oss K = 2880 is 23 chunks: parts of 12 and 11.
__device__ __forceinline__ void k_part_range(int C, int part, int ksplit, int& cb, int& ce,
                                             int& Cp) {
  Cp = ((C + ksplit - 1) / ksplit + 3) & ~3;
  cb = part * Cp;
  ce = min(C, cb + Cp);
}

}  // namespace moe
