// mx4_moe_gemm: routed-expert MXFP4 projection for prefill, on bf16 MFMA with fp32 accumulation;
// mx4_moe_gemm_mx8: the same pipeline over MXFP8 activation rows, on the MX-scaled MFMA.
//
// Sources: PR #3579 "dasLLAMA gpt-oss arc", Metal fusion-lane commit (the grouped expert matmul
// over the buckets starts its accumulator tiles from the expert's bias row instead of running a
// separate bias pass; the SwiGLU-OAI epilogue skips ghost rows past the last padded bucket end);
// PR #3558 "dasLLAMA: dig the last two board reds green", section "gpt-oss: mx4 kernels to the
// lab-winning shape" (the matmul's weight stage: 16-byte block loads, e2m1 table decode, e8m0
// applied arithmetically).
//
// gfx950 mapping. One workgroup (8 wavefronts) owns one expert and one slice of weight rows and
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
//  * The K loop is a software pipeline: chunk c + 3 of the activations is copied into LDS by
//    LDS-DMA buffer loads (no registers) at the start of iteration c, and chunk c + 4 of the
//    weights is loaded into the register ring slot that chunk c has just used, at its end, so
//    the slot is refilled in place (no register copies across the loop, whose waits would drain
//    the pipeline). Vector loads complete in issue order and every iteration issues the same
//    loads (chunks past K re-read the last one; their compute is skipped), so one wait for
//    "everything but the last two iterations' loads and one weight chunk" at the top of
//    iteration c covers both the weights and the activations of chunk c. A barrier per chunk
//    publishes the activation chunk to all wavefronts and frees the LDS buffer (of 4) that the
//    iteration's DMA overwrites.
//  * Activation rows are gathered through a_row (row_tok) by the DMA, 128 k (256 B) per row
//    per chunk, into an XOR-swizzled LDS layout (16-byte piece q of row m at slot
//    q ^ gemm_swz16(m)), so the 1 KB B-fragment reads of 16 consecutive rows run at the LDS's
//    full rate; every B fragment feeds the wavefront's 2 (SwiGLU) or 3 weight tiles.
//  * Accumulators start at the bias of their weight row. Token tiles past the expert's count are
//    never computed; rows past the count are never stored. Experts with no rows exit at once.
//  * SwiGLU mode pairs gate tiles with the matching up tiles in the same wavefront, so the
//    epilogue is register-local and only bf16 h leaves the kernel.
//  * MXFP8 variant: activation rows are E4M3 bytes (128 B per row per chunk, swizzled over 8
//    pieces by gemm_swz8) and v_mfma_scale_f32_16x16x128_f8f6f4 takes the lane's 16-byte MX
//    block unchanged as its A operand (32 e2m1 values: weight row lr, block 4c + lg), with the
//    block's e8m0 byte as the A scale, so nothing is decoded in registers. Its B operand holds
//    k 16*lg..16*lg+15 and 64+16*lg..64+16*lg+15 of the token column (the instruction's operand
//    layout on gfx950, established by a one-wavefront layout check against the exact product),
//    and the B scale is the activation block's e8m0 byte, from the pass's scale rows staged in
//    LDS. One MFMA per weight tile, token tile and chunk replaces 4 bf16 MFMAs and 4 converts.
#include "gemv_core.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kGmWaves = 8;              // 2 wavefronts per SIMD
constexpr int kXcds = 8;                 // XCDs of an MI355X, each with its own L2
constexpr int kGmThreads = 64 * kGmWaves;
constexpr int kGmMaxWT = 6;              // weight tiles (16 rows each) per wavefront, at most
// SwiGLU: 2 tiles (16 gate rows + the matching 16 up rows); plain: 3 tiles (384 rows per
// workgroup), which at gpt-oss shapes makes the down projection's grid a whole number of
// rounds over the 256 CUs (2880 / 384 -> 8 workgroups per expert)
__host__ __device__ constexpr int gemm_wt(int act) { return act == MOE_ACT_SWIGLU_OAI ? 2 : 3; }
constexpr int kGmTT = 8;                 // token tiles (16 rows each) per pass: 128 routed rows
constexpr int kGmChunkK = 128;           // k per chunk = 4 MX blocks
// activation bytes per row per chunk: bf16 rows, or MXFP8 rows (E4M3 bytes; their e8m0 scales
// are staged separately, once per pass)
__host__ __device__ constexpr int gemm_row_bytes(bool mx8) { return mx8 ? kGmChunkK : 2 * kGmChunkK; }

// weight chunks in flight (register ring slots): 4 with 2 tiles per wavefront, 3 with 3 tiles
// (registers); the activation chunks are issued 3 ahead either way
__host__ __device__ constexpr int gemm_wring(int wt) { return wt == 2 ? 4 : 3; }
constexpr int kGmXRing = 4;              // activation chunk buffers in LDS (3 chunks ahead)
// LDS of one activation chunk of a pass with NTT token tiles
__host__ __device__ constexpr int gemm_buf_bytes(int ntt, bool mx8) {
  return ntt * 16 * gemm_row_bytes(mx8);
}
// after the activation ring: 1 KB that the DMA of wavefronts without a share of a chunk writes;
// MXFP8 passes then stage the e8m0 scale rows of their 128 routed rows
// MXFP8 passes hold two super-chunks of activations (a super-chunk = one weight ring's worth of
// chunks, at most 4) instead of a ring of 4 chunks: the same 128 KB
constexpr int kGmScMax = 4;
__host__ __device__ constexpr int gemm_dummy_off(bool mx8) {
  return (mx8 ? 2 * kGmScMax : kGmXRing) * gemm_buf_bytes(kGmTT, mx8);
}
// LDS pitch of a staged scale row: fixed, so that a token tile's offset is an immediate
constexpr int kGmScalePitch = MOE_MX8_GEMM_MAX_K / 32;
constexpr int kMxWaves = 8;              // MXFP8 variant: 2 wavefronts per SIMD as well
// MXFP8 passes, after the staged scale rows: the per-wavefront h block maxima that the MXFP8
// epilogue exchanges (one word per wavefront and routed row)
__host__ __device__ constexpr int gemm_amax_off() {
  return gemm_dummy_off(true) + 1024 + kGmTT * 16 * kGmScalePitch;
}
__host__ __device__ constexpr int gemm_lds_bytes(bool mx8) {
  return mx8 ? gemm_amax_off() + kMxWaves * kGmTT * 16 * 4 : gemm_dummy_off(false) + 1024;
}
// 16-byte piece q of routed row m of an MXFP8 chunk sits at slot q ^ gemm_swz8(m) of the row's
// 128 bytes: the B-fragment reads of 16 consecutive rows at one q then touch 16 different
// 16-byte bank groups (8 different ones for rows m and m + 8 apart in the low bit)
__device__ __forceinline__ int gemm_swz8(int m) { return (m & 7) ^ ((m >> 3) & 1); }
// 16-byte piece q of routed row m of a bf16 chunk (256 bytes) sits at slot q ^ gemm_swz16(m):
// m % 16 rotated left by one bit. Measured with the LDS counters on gfx950 (one ds_read_b128
// per lane, lane (r, g) reading piece 4g + i of row r, rows 256 bytes apart): this mask costs the
// 4 LDS cycles of a contiguous 1 KB read, while the plain mask m % 16 costs 8, half of them
// bank-conflict stalls.
__device__ __forceinline__ int gemm_swz16(int m) { return ((m << 1) & 14) | ((m >> 3) & 1); }

// Everything one pass over up to 16*NTT routed rows of one expert needs.
struct GemmCtx {
  const int32_t* a_row;
  const float* bias;
  void* out;
  const uint8_t* a_scale;   // MXFP8 activation scale rows (pitch spa), else unused
  uint8_t* xs;              // the workgroup's LDS
  uint8_t* out_scale;       // MOE_ACT_SWIGLU_OAI_MX8: e8m0 rows of h (pitch spo)
  int spo;
  __amdgpu_buffer_rsrc_t rq, rs, ra, ras;
  int e, N, K, KB, C, klast, row0, p0, live, F, spa;
  int tid, lr, lg;
  float alpha, limit;
  int tile_base[kGmMaxWT];
  int rows_in[kGmMaxWT];
  uint32_t wo[kGmMaxWT], wol[kGmMaxWT], so[kGmMaxWT];
  uint32_t sg[kGmMaxWT];   // the lane's row in a scale group (16 bytes: 4 chunks)
};

// Activation row that DMA slot m of the pass reads (a_row, or CSR order when a_row is NULL).
// Slots without a routed row (m >= live) read the pass's first row and are pointed past the
// resource by the caller: every lane loads, with no branch, so a wavefront issues all of its
// row-id loads at once and the pass start waits for them together.
__device__ __forceinline__ uint32_t gemm_src_row(const GemmCtx& g, int m, bool ok) {
  const int r = g.row0 + g.p0 + (ok ? m : 0);
  return g.a_row ? (uint32_t)g.a_row[r] : (uint32_t)r;
}

// Bias seeds of the lane's rows 4*lg..4*lg+3 of each weight tile (0 past the tile's rows or
// without a bias); the loads are unconditional (clamped to row N - 1), so they issue together.
template <int WT>
__device__ __forceinline__ void gemm_bias(const GemmCtx& g, float (&b)[WT][4]) {
#pragma unroll
  for (int t = 0; t < WT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) b[t][i] = 0.0f;
  if (!g.bias) return;
  const float* be = g.bias + (size_t)g.e * g.N;
#pragma unroll
  for (int t = 0; t < WT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g.lg + i;
      const float v = be[min(g.tile_base[t] + r, g.N - 1)];
      b[t][i] = r < g.rows_in[t] ? v : 0.0f;
    }
}

// Epilogue of a pass: lane holds rows 4*lg..4*lg+3 of each weight tile for token column lr.
// SwiGLU: tiles [0, WT/2) are gate rows, tile t + WT/2 the matching up rows.
template <int ACT, int NTT, int WT>
__device__ __forceinline__ void gemm_epilogue(const GemmCtx& g, const f32x4_t (&acc)[WT][NTT]) {
  constexpr bool swiglu = (ACT == MOE_ACT_SWIGLU_OAI);
  constexpr int kGmWT = WT;
  const int lr = g.lr, lg = g.lg;
  if constexpr (ACT == MOE_ACT_SWIGLU_OAI_MX8) {
    // MXFP8 rows of h. A wavefront holds 16 h columns [jb, jb + 16) (gate tile 0, up tile 1),
    // rows 4*lg..4*lg+3 of them per lane; an MX block of 32 columns is the work of wavefronts
    // 2i and 2i + 1. The block maximum per token row: over the lane's 4 values, the 4 lanes of
    // the token column (two cross-lane steps), then the partner wavefront's maximum through LDS.
    // Values are the bf16-rounded SwiGLU-OAI outputs, scaled and encoded as mx8_quantize does.
    static_assert(WT == 2, "16 columns per wavefront, a block per wavefront pair");
    const int jb = g.tile_base[0];
    const int nblk = g.F >> 5;
    const int wave = g.tid >> 6;
    uint32_t* const amax_w = reinterpret_cast<uint32_t*>(g.xs + gemm_amax_off());
    uint32_t hp[NTT][2];   // the lane's 4 bf16 values, two per word
    uint32_t amax[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      uint32_t a = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t hb =
            f32_to_bf16_bits(swiglu_oai(acc[0][tt][i], acc[1][tt][i], g.alpha, g.limit));
        a = max(a, hb & 0x7FFFu);
        if (i % 2 == 0) hp[tt][i / 2] = hb;
        else hp[tt][i / 2] |= hb << 16;
      }
      a = max(a, (uint32_t)__shfl_xor((int)a, 16));
      a = max(a, (uint32_t)__shfl_xor((int)a, 32));
      amax[tt] = a;
      if (lg == 0) amax_w[wave * (kGmTT * 16) + tt * 16 + lr] = a;
    }
    __syncthreads();   // block maxima published; every wavefront is past the K loop
    // codes and scale bytes go through LDS (the activation buffers, free now) and out as whole
    // rows: stored straight from the lanes, 4-byte code pieces and single scale bytes each
    // cost a whole write granule (3x the bytes in HBM writes)
    constexpr int kPitch = 144;   // 128 code bytes + 16: rows 16 bytes apart in the banks
    uint8_t* const stage = g.xs;
    uint8_t* const stage_s = stage + kGmTT * 16 * kPitch;   // 4 scale bytes per row
    const int jb0 = jb - wave * 16;                          // the slice's first column
    const int cols = min(128, g.F - jb0);                    // a multiple of 32
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const int m = tt * 16 + lr;
      const uint32_t a = max(amax[tt], amax_w[(wave ^ 1) * (kGmTT * 16) + m]);
      const uint32_t sbyte = mx8_scale_byte(a);
      const float inv = mx8_inv_scale(sbyte);
      uint32_t pk = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pk |= e4m3_rne_sat(bf16_bits_to_f32((hp[tt][i / 2] >> (16 * (i % 2))) & 0xFFFFu) * inv)
              << (8 * i);
      *reinterpret_cast<uint32_t*>(stage + m * kPitch + wave * 16 + 4 * lg) = pk;
      if (lg == 0 && (wave & 1) == 0) stage_s[m * 4 + (wave >> 1)] = (uint8_t)sbyte;
    }
    __syncthreads();
    const int tid = g.tid;
    for (int idx = tid; idx < NTT * 16 * 8; idx += 8 * 64) {   // 8 lanes x 16 bytes per row
      const int m = idx >> 3, q = idx & 7;
      if (m < g.live && q * 16 < cols) {
        const size_t r = (size_t)(g.row0 + g.p0 + m);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(g.out) + r * g.F + jb0 + q * 16) =
            *reinterpret_cast<const uint4*>(stage + m * kPitch + q * 16);
      }
    }
    for (int m = tid; m < NTT * 16; m += 8 * 64) {   // the row's scale bytes of this slice
      if (m >= g.live) continue;
      uint8_t* srow = g.out_scale + (size_t)(g.row0 + g.p0 + m) * g.spo;
      const int b0 = jb0 >> 5, nb = cols >> 5;
      if (nb == 4) {
        *reinterpret_cast<uint32_t*>(srow + b0) = *reinterpret_cast<const uint32_t*>(stage_s + m * 4);
      } else {
        for (int b = 0; b < nb; ++b) srow[b0 + b] = stage_s[m * 4 + b];
      }
      if (b0 + nb == nblk)
        for (int p = nblk; p < g.spo; ++p) srow[p] = 0;   // the row's padding
    }
    return;
  }
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int m = tt * 16 + lr;
    if (m >= g.live) continue;
    const size_t r = (size_t)(g.row0 + g.p0 + m);
    if (swiglu) {
#pragma unroll
      for (int t = 0; t < WT / 2; ++t) {
        const int j0 = g.tile_base[t] + 4 * lg;
        uint16_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          h[i] = (uint16_t)f32_to_bf16_bits(
              swiglu_oai(acc[t][tt][i], acc[t + WT / 2][tt][i], g.alpha, g.limit));
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

// One pass with NTT live token tiles over bf16 activations, on bf16 MFMA (compile-time NTT, so
// the MFMA loop is straight-line code and LDS reads can be scheduled ahead of the MFMAs).
template <int ACT, int NTT>
__device__ __forceinline__ void gemm_pass(const GemmCtx& g, uint8_t* __restrict__ xs) {
  constexpr bool swiglu = (ACT == MOE_ACT_SWIGLU_OAI);
  constexpr int kGmWT = gemm_wt(ACT);
  constexpr int ROWB = gemm_row_bytes(false);
  constexpr int PIECES = ROWB / 16;          // 16-byte pieces per row per chunk
  constexpr int BUF = gemm_buf_bytes(NTT, false);
  constexpr int KBS = BUF / 1024;            // 1 KB DMA instructions per chunk
  // DMA instructions per wavefront per chunk: the chunk's KBS KB split over the wavefronts,
  // every wavefront issuing the same count (surplus ones copy zeros into a dummy KB) so that
  // the vector-memory counter waits below are exact for each of them
  constexpr int NX = (KBS + kGmWaves - 1) / kGmWaves;
  constexpr int LOADS = NX + 2 * kGmWT;   // vector-memory instructions per wavefront per chunk
  static_assert(2 * kGmWT + 2 * LOADS <= 63, "vmcnt range");
  const int C = g.C;
  const int lr = g.lr, lg = g.lg;
  const int lane = g.tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(g.tid >> 6);   // uniform: LDS-DMA base
  const int dummy = gemm_dummy_off(false);

  // weight fetch of chunk c into a ring slot. Chunks past K re-read the last chunk (their
  // compute is skipped), so every chunk issues the same loads and only the last one differs
  // (its narrower row pitch): one uniform select per offset, no branches.
  auto load_w = [&](int c, u32x4_t (&dq)[kGmWT], uint32_t (&dx)[kGmWT]) {
    const int cc = min(c, C - 1);
    const bool last = cc == C - 1;
    const uint32_t cq = (uint32_t)cc * g.N * (kChunkBlocks * 16);
    // scale byte of block 4c + lg: byte 4 (c % 4) + lg of the row's 16 bytes in group c / 4
    const uint32_t cs = (uint32_t)(cc >> 2) * g.N * 16 + (uint32_t)(cc & 3) * kChunkBlocks;
#pragma unroll
    for (int t = 0; t < kGmWT; ++t) {
      dq[t] = buf_load16(g.rq, last ? g.wol[t] : g.wo[t], cq);
      dx[t] = buf_load8(g.rs, g.so[t], cs);
    }
  };

  // activation DMA: instruction i of this wavefront covers 16-byte slots p = j*64 + lane,
  // j = wave + 8*i, i.e. routed row m = p / 16 of the pass and swizzled slot p % 16, which
  // holds the row's piece q = (p % 16) ^ gemm_swz16(m) of the chunk
  uint32_t xo[NX], xol[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int p = (wave + kGmWaves * i) * 64 + lane;
    const int m = p / PIECES;
    const int q = (p % PIECES) ^ gemm_swz16(m);
    const bool ok = m < g.live && wave + kGmWaves * i < KBS;
    const uint32_t src = gemm_src_row(g, m, ok);
    const uint32_t off = ok ? src * (uint32_t)g.K * 2 + q * 16 : kOOB;
    xo[i] = off;
    // the last chunk may be narrower than 128 k
    xol[i] = (q * 8 < g.klast) ? off : kOOB;
  }
  auto load_x = [&](int c) {
    const int cc = min(c, C - 1);
    const bool last = cc == C - 1;
    const int dst = (c % kGmXRing) * BUF;
    const uint32_t ck = (uint32_t)cc * ROWB;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int j = wave + kGmWaves * i;   // uniform
      const int d = j < KBS ? dst + j * 1024 : dummy;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          g.ra, (__attribute__((address_space(3))) void*)(xs + d), 16, last ? xol[i] : xo[i], ck,
          0, 0);
    }
  };

  f32x4_t acc[kGmWT][NTT];
  {
    float b[kGmWT][4];
    gemm_bias<kGmWT>(g, b);
#pragma unroll
    for (int t = 0; t < kGmWT; ++t)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) acc[t][tt] = f32x4_t{b[t][0], b[t][1], b[t][2], b[t][3]};
  }

  constexpr int kGmWRing = gemm_wring(kGmWT);
  // B fragments in flight (LDS reads ahead of their MFMAs), on the SwiGLU passes of up to
  // kBRingTT token tiles; the plain passes (3 weight tiles) have no registers to spare for it
  constexpr int kBD = 4;
  constexpr int kBRingTT = swiglu ? 6 : 0;
  u32x4_t wq[kGmWRing][kGmWT];
  uint32_t wx[kGmWRing][kGmWT];

  __syncthreads();  // the previous pass is done with the LDS buffers
  // prologue, in the steady state's issue order (W0 X0 W1 X1 W2 X2 W3 with a ring of 4;
  // X0 W0 X1 W1 X2 W2 with a ring of 3)
  // (issue_fence, not only a scheduling barrier: the plain weight loads would otherwise sink
  // below the DMA copies, and the compiler's wait before the first MFMAs, merged into the loop
  // header, would then hold every later chunk for a younger load than it needs)
  issue_fence();
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (kGmWRing == 4 && c < kGmWRing) {
      load_w(c, wq[c], wx[c]);
      issue_fence();
    }
    if (c < kGmXRing - 1) {
      load_x(c);
      issue_fence();
    }
    if (kGmWRing == 3 && c < kGmWRing) {
      load_w(c, wq[c], wx[c]);
      issue_fence();
    }
  }

  const int swz = gemm_swz16(lr);   // m % 16 == lr for every token tile
  // a do-while: C >= 1, and a loop the compiler may skip lets it sink the prologue's weight
  // loads into the loop's entry block, below the DMA copies
  int c0 = 0;
  do {
#pragma unroll
    for (int sl = 0; sl < kGmWRing; ++sl) {
      const int c = c0 + sl;
      // issued after X(c): one weight chunk, then two iterations' X and W -> waiting until only
      // those are outstanding completes X(c) (and W(c) with the ring of 4, issued before it;
      // with the ring of 3 the register dependency makes the compiler wait for W(c))
      // A bare s_barrier, not __syncthreads(): its fence would also wait for the DMA copies of
      // the chunks still in flight. Here the wait above has landed this wavefront's share of
      // X(c) in LDS, and every wavefront consumed its LDS reads of chunk c - 1 (in its MFMAs)
      // before arriving, so after the barrier X(c) is complete and buffer (c - 1) % 4 is free.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kGmWT + 2 * LOADS));
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      load_x(c + kGmXRing - 1);
      __builtin_amdgcn_sched_barrier(0);
      if (c < C) {
        const uint8_t* xb = xs + (c % kGmXRing) * BUF;
        float cs[kGmWT];
#pragma unroll
        for (int t = 0; t < kGmWT; ++t) cs[t] = e8m0_scale_operand(wx[sl][t]);
        auto read_b = [&](int i, int tt) {
          const int m = tt * 16 + lr;   // m % 16 == lr
          return *reinterpret_cast<const bf16x8_t*>(xb + (m * 16 + ((lg * 4 + i) ^ swz)) * 16);
        };
        if constexpr (NTT <= kBRingTT) {
          // the chunk's steps st = (k substep i, token tile tt), i major; the B fragment of
          // step st is read from LDS kBD steps ahead into a ring, so each read has kBD - 1
          // steps of MFMAs to land (read at use, it was waited for with two MFMAs in flight)
          constexpr int NS = 4 * NTT;
          bf16x8_t Bq[kBD];
#pragma unroll
          for (int st = 0; st < kBD && st < NS; ++st) Bq[st] = read_b(st / NTT, st % NTT);
          // A of substep i + 1 is decoded after the first step's MFMAs of substep i (a second
          // set of A registers), so the converts overlap the matrix core instead of holding up
          // the substep's first MFMA
          bf16x8_t A[2][kGmWT];
#pragma unroll
          for (int t = 0; t < kGmWT; ++t) A[0][t] = dequant8(wq[sl][t][0], cs[t]);
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const int i = st / NTT, tt = st % NTT;
#pragma unroll
            for (int t = 0; t < kGmWT; ++t)
              acc[t][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i & 1][t], Bq[st % kBD],
                                                                  acc[t][tt], 0, 0, 0);
            if (st + kBD < NS) Bq[st % kBD] = read_b((st + kBD) / NTT, (st + kBD) % NTT);
            if (tt == 0 && i < 3) {
#pragma unroll
              for (int t = 0; t < kGmWT; ++t)
                A[(i + 1) & 1][t] = dequant8(wq[sl][t][i + 1], cs[t]);
            }
            // keeps each read at its step (the scheduler would sink them to their use)
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            bf16x8_t A[kGmWT];
#pragma unroll
            for (int t = 0; t < kGmWT; ++t) A[t] = dequant8(wq[sl][t][i], cs[t]);
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
              const bf16x8_t B = read_b(i, tt);
#pragma unroll
              for (int t = 0; t < kGmWT; ++t)
                acc[t][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t], B, acc[t][tt], 0, 0, 0);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_w(c + kGmWRing, wq[sl], wx[sl]);   // refill the slot chunk c used, in place
      __builtin_amdgcn_sched_barrier(0);
    }
    c0 += kGmWRing;
  } while (c0 < C);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // no LDS-DMA write outlives the pass

  gemm_epilogue<ACT, NTT, kGmWT>(g, acc);
}

// MXFP8 pass on the MX-scaled MFMA. The arithmetic per byte is small here (no decode, one MFMA
// per 16x16x128 tile product), so the pass is bound by keeping weight bytes in flight while the
// matrix core works: 8 wavefronts, 2 per SIMD (one waits on memory while the other issues
// MFMAs), each with a ring of weight chunks (SwiGLU: 8 chunks of 2 tiles, 16 KB, or 4 chunks
// with the MXFP8 epilogue, whose extra live state would otherwise spill to scratch memory;
// plain: 4 chunks of 3 tiles, 12 KB). The activations move in super-chunks of 4 chunks, double-buffered in LDS,
// so the workgroup meets at a barrier once per 4 chunks; between barriers each wavefront
// streams its own weights. B operands are read from LDS one token tile ahead of their MFMAs
// (all of a chunk's at once would hold 8 x 8 registers).
//  * Issue order per super-chunk: the DMA of the next super-chunk, then after each chunk's MFMAs
//    the weight chunk WRING ahead into the slot just used. At the top of super-chunk s, waiting
//    until only the 4 weight chunks issued after its DMA are outstanding lands that DMA (loads
//    complete in issue order); the barrier makes it every wavefront's and frees the half that
//    the next DMA overwrites. The weights of each chunk are waited for by the compiler
//    (register dependencies).
constexpr int kMxThreads = 64 * kMxWaves;
constexpr int kMxSC = 4;   // chunks per activation super-chunk
__host__ __device__ constexpr int mx_wt(int act) { return act != MOE_ACT_NONE ? 2 : 3; }
__host__ __device__ constexpr int mx_wring(int act) { return act == MOE_ACT_SWIGLU_OAI_MX8 ? 4 : act != MOE_ACT_NONE ? 8 : 4; }
constexpr int SRING_MAX = 2;   // scale groups in flight, at most (mx_wring / kMxSC)
static_assert(gemm_dummy_off(true) == 2 * kMxSC * gemm_buf_bytes(kGmTT, true), "MX LDS layout");

template <int ACT, int NTT>
__device__ __forceinline__ void gemm_pass_mx8(const GemmCtx& g, uint8_t* __restrict__ xs) {
  constexpr int WT = mx_wt(ACT);
  constexpr int WRING = mx_wring(ACT);
  constexpr int SC = kMxSC;
  constexpr int ITER = WRING > SC ? WRING : SC;   // chunks per loop trip (slots compile-time)
  static_assert(ITER % SC == 0 && ITER % WRING == 0, "loop trip");
  constexpr int ROWB = gemm_row_bytes(true);      // 128 E4M3 bytes per row per chunk
  constexpr int PIECES = ROWB / 16;
  constexpr int BUF = gemm_buf_bytes(NTT, true);
  constexpr int KBS = BUF / 1024;                 // 1 KB DMA instructions per chunk
  constexpr int NX = (KBS + kMxWaves - 1) / kMxWaves;
  static_assert(WT * (WRING + SRING_MAX) + 4 * SC <= 63, "loads in flight per wavefront");
  const int C = g.C;
  const int lr = g.lr, lg = g.lg;
  const int lane = g.tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(g.tid >> 6);
  const int dummy = gemm_dummy_off(true);

  // nibbles of chunk c into a ring slot (chunks past K re-read the last one)
  auto load_w = [&](int c, u32x4_t (&dq)[WT]) {
    const int cc = min(c, C - 1);
    const bool last = cc == C - 1;
    const uint32_t cq = (uint32_t)cc * g.N * (kChunkBlocks * 16);
#pragma unroll
    for (int t = 0; t < WT; ++t) dq[t] = buf_load16(g.rq, last ? g.wol[t] : g.wo[t], cq);
  };
  // e8m0 scales of the SC chunks of super-chunk s, one 16-byte load per tile: the scale of
  // chunk s*SC + j for this lane is byte lg of dword j (super-chunks past K re-read the last)
  static_assert(SC == 4, "a 16-byte scale load covers 4 chunks");
  const int S_last = (C - 1) / SC;
  auto load_s = [&](int s, u32x4_t (&ds)[WT]) {
    const uint32_t off = (uint32_t)min(s, S_last) * g.N * 16;
#pragma unroll
    for (int t = 0; t < WT; ++t) ds[t] = buf_load16(g.rs, g.sg[t], off);
  };

  // activation DMA slots of this wavefront: 16-byte slot p = (wave + 4*i)*64 + lane of a chunk
  // buffer holds piece (p % 8) ^ gemm_swz8(m) of routed row m = p / 8
  uint32_t xo[NX], xol[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int p = (wave + kMxWaves * i) * 64 + lane;
    const int m = p / PIECES;
    const int q = (p % PIECES) ^ gemm_swz8(m);
    const bool ok = m < g.live && wave + kMxWaves * i < KBS;
    const uint32_t src = gemm_src_row(g, m, ok);
    const uint32_t off = ok ? src * (uint32_t)g.K + q * 16 : kOOB;
    xo[i] = off;
    xol[i] = (q * 16 < g.klast) ? off : kOOB;
  }
  // super-chunk s into LDS half s % 2 (chunks past K re-read the last one)
  auto load_x_super = [&](int s) {
#pragma unroll
    for (int j = 0; j < SC; ++j) {
      const int cc = min(s * SC + j, C - 1);
      const bool last = cc == C - 1;
      const int dst = ((s & 1) * SC + j) * BUF;
      const uint32_t ck = (uint32_t)cc * ROWB;
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        const int jj = wave + kMxWaves * i;
        const int d = jj < KBS ? dst + jj * 1024 : dummy;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            g.ra, (__attribute__((address_space(3))) void*)(xs + d), 16, last ? xol[i] : xo[i],
            ck, 0, 0);
      }
    }
  };

  f32x4_t acc[WT][NTT];
#pragma unroll
  for (int t = 0; t < WT; ++t) {
    float b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * lg + i;
      b[i] = (g.bias && r < g.rows_in[t]) ? g.bias[(size_t)g.e * g.N + g.tile_base[t] + r] : 0.0f;
    }
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[t][tt] = f32x4_t{b[0], b[1], b[2], b[3]};
  }
  constexpr int SRING = WRING / SC;   // scale groups in flight
  u32x4_t wq[WRING][WT];
  u32x4_t ws[SRING][WT];

  __syncthreads();  // the previous pass is done with the LDS buffers
  // the e8m0 scale rows of the pass's routed rows, row m at xsc + m * kGmScalePitch, its 16-byte
  // piece p at slot p ^ gemm_swz8(m) (rows 128 bytes apart would otherwise put the scale bytes
  // that 16 consecutive rows read together into one or two banks)
  uint8_t* const xsc = xs + dummy + 1024;
  static_assert(kGmScalePitch == 128, "8 pieces per staged scale row");
  // 1 KB = 8 rows per instruction, at most 2 per wavefront; row ids loaded together first
  constexpr int NSC = (NTT * 2 + kMxWaves - 1) / kMxWaves;
  uint32_t soff[NSC];
#pragma unroll
  for (int i = 0; i < NSC; ++i) {
    const int m = (wave + kMxWaves * i) * 8 + lane / 8;
    const int piece = (lane % 8) ^ gemm_swz8(m);
    const bool ok = m < g.live && piece * 16 < g.spa;
    const uint32_t src = gemm_src_row(g, m, ok);
    soff[i] = ok ? src * (uint32_t)g.spa + piece * 16 : kOOB;
  }
#pragma unroll
  for (int i = 0; i < NSC; ++i) {
    const int j = wave + kMxWaves * i;   // uniform
    if (j < NTT * 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          g.ras, (__attribute__((address_space(3))) void*)(xsc + j * 1024), 16, soff[i], 0, 0, 0);
  }
  issue_fence();
  load_x_super(0);
  issue_fence();
#pragma unroll
  for (int j = 0; j < WRING; ++j) {
    if (j % SC == 0) load_s(j / SC, ws[j / SC]);
    load_w(j, wq[j]);
    issue_fence();
  }

  const int swz = gemm_swz8(lr);
  int cb = 0;   // first chunk of the loop trip
  do {          // a do-while: C >= 1 (see gemm_pass)
#pragma unroll
    for (int sub = 0; sub < ITER / SC; ++sub) {
      const int s = cb / SC + sub;
      // after the DMA of super-chunk s: SC nibble chunks and one scale group
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(WT * SC + WT));
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      load_x_super(s + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < SC; ++j) {
        const int slot = (sub * SC + j) % WRING;
        const int gslot = sub % SRING;
        const int c = s * SC + j;
        if (c < C) {
          const uint8_t* xb = xs + ((s & 1) * SC + j) * BUF;
          const bool kb_live = 4 * c + lg < g.KB;
          int sa[WT];   // the MFMA reads the low byte
#pragma unroll
          for (int t = 0; t < WT; ++t) sa[t] = kb_live ? (int)(ws[gslot][t][j] >> (8 * lg)) : 0;
          const uint8_t* xb0 = xb + lr * ROWB + ((lg ^ swz) << 4);
          const uint8_t* xb1 = xb + lr * ROWB + (((4 + lg) ^ swz) << 4);
          // scale byte 4c + lg of row m: piece c / 4, byte 4 (c % 4) + lg (swizzled as staged)
          const uint8_t* sbp =
              xsc + lr * kGmScalePitch + (((c >> 2) ^ swz) << 4) + 4 * (c & 3) + lg;
          auto read_b = [&](int tt, i32x8_t& B, int& sb) {
            const u32x4_t b0 = *reinterpret_cast<const u32x4_t*>(xb0 + tt * 16 * ROWB);
            const u32x4_t b1 = *reinterpret_cast<const u32x4_t*>(xb1 + tt * 16 * ROWB);
            const int sv = sbp[tt * 16 * kGmScalePitch];   // read always, then select: no branch
            sb = kb_live ? sv : 0;
            B = i32x8_t{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                        (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
          };
          i32x8_t Bn;
          int sbn;
          read_b(0, Bn, sbn);
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) {
            const i32x8_t B = Bn;
            const int sb = sbn;
            if (tt + 1 < NTT) read_b(tt + 1, Bn, sbn);
#pragma unroll
            for (int t = 0; t < WT; ++t) {
              const i32x8_t A = {(int)wq[slot][t][0], (int)wq[slot][t][1], (int)wq[slot][t][2],
                                 (int)wq[slot][t][3], 0, 0, 0, 0};
              acc[t][tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  A, B, acc[t][tt], kMfmaFmtFp4, kMfmaFmtFp8, 0, sa[t], 0, sb);
            }
            issue_fence();   // B of token tile tt + 1 only: LDS reads stay one tile ahead
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // refill in place: the nibble slot chunk c used, and after the super-chunk's last chunk
        // its scale group (the same load counts in every super-chunk)
        load_w(c + WRING, wq[slot]);
        if (j == SC - 1) load_s(s + SRING, ws[gslot]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    cb += ITER;
  } while (cb < C);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // no LDS-DMA write outlives the pass

  gemm_epilogue<ACT, NTT, WT>(g, acc);
}

__host__ __device__ constexpr int gemm_threads(bool mx8) { return mx8 ? kMxThreads : kGmThreads; }
// Tile order by expert cost across the XCDs (bf16 activations, E <= 64); the MXFP8 variant
// measured slower with it and keeps the id order
__host__ __device__ constexpr bool gemm_balanced(int E, bool mx8) { return !mx8 && E <= kWave; }

// Both variants: 8 wavefronts, 2 per SIMD (256 registers each)
template <int ACT, bool MX8>
__global__ void __launch_bounds__(gemm_threads(MX8), 1)
gemm_kernel(const void* __restrict__ a, const uint8_t* __restrict__ a_scale, int a_rows,
            const int32_t* __restrict__ a_row, const uint8_t* __restrict__ q,
            const uint8_t* __restrict__ s, const float* __restrict__ bias,
            const int32_t* __restrict__ counts, const int32_t* __restrict__ basep, int E, int N,
            int K, float alpha, float limit, void* __restrict__ out,
            uint8_t* __restrict__ out_scale, int nbx, int nslots, int per_xcd) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  // XCD-aware tile order: the hardware deals workgroup ids to the 8 XCDs round robin, so id L
  // runs on XCD L % 8, and the L / 8-th workgroup of an XCD takes its tile (bx fastest), so each
  // XCD works through whole experts and its L2 holds the activation rows of the one or two
  // experts it is on instead of every expert's.
  //  * E <= 64: experts go to XCDs by cost, so that no XCD is left with the heavy ones while the
  //    others idle. Every workgroup ranks the live experts by cost (token tiles plus two per
  //    pass, for its set-up and drain; ties by id) from the counts, the same ranking everywhere,
  //    and rank r is position r / 8 on XCD r % 8, or 7 - r % 8 in odd rounds (a snake); heavy
  //    experts come first on each XCD, light ones fill the tail.
  //  * E > 64: live experts in id order, each XCD a contiguous run of tiles.
  const int L = (int)blockIdx.x;
  const int xcd = L % kXcds, idx = L / kXcds;
  const int lane0 = (int)(threadIdx.x & 63);
  // each lane: count and padded base of expert lane, loaded together
  const int c64 = lane0 < E ? counts[lane0] : 0;
  const int b64 = lane0 < E ? basep[lane0] : 0;
  int e, bxi, row0, cnt;
  if (gemm_balanced(E, MX8)) {
    const int pos = idx / nbx;
    bxi = idx - pos * nbx;
    const int passes = (c64 + kGmTT * 16 - 1) / (kGmTT * 16);
    const int cost = c64 > 0 ? (c64 + 15) / 16 + 2 * passes : 0;
    // every expert's cost to this wavefront's own 256 bytes of the LDS (unused before the first
    // pass), then eight compares per step against broadcast reads of it, independent of each
    // other (a v_readlane broadcast per expert waits for its scalar register every step)
    int* const cl = reinterpret_cast<int*>(xs) + (threadIdx.x >> 6) * kWave;
    cl[lane0] = cost;
    int rank = 0;
    for (int j0 = 0; j0 < E; j0 += 8) {
      const int4 a = *reinterpret_cast<const int4*>(cl + j0);
      const int4 b = *reinterpret_cast<const int4*>(cl + j0 + 4);
      const int cj[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int u = 0; u < 8; ++u)
        rank += (int)((j0 + u < E) & ((cj[u] > cost) | ((cj[u] == cost) & (j0 + u < lane0))));
    }
    const int r = kXcds * pos + ((pos & 1) ? kXcds - 1 - xcd : xcd);
    const uint64_t hit = __ballot(cost > 0 && rank == r);
    if (hit == 0) return;   // uniform over the workgroup: fewer live experts than positions
    e = __ffsll((unsigned long long)hit) - 1;
    row0 = __builtin_amdgcn_readlane(b64, e);
    cnt = __builtin_amdgcn_readlane(c64, e);
  } else {
    const int v = xcd * per_xcd + idx;
    if (v >= nbx * nslots) return;
    bxi = v % nbx;
    e = wave_slot_expert(counts, E, v / nbx, c64);
    if (e < 0) return;   // uniform over the workgroup: fewer live experts than slots
    row0 = basep[e];
    cnt = counts[e];
  }
  constexpr bool swiglu = (ACT != MOE_ACT_NONE);
  GemmCtx g;
  g.a_row = a_row;
  g.bias = bias;
  g.out = out;
  g.a_scale = a_scale;
  g.out_scale = out_scale;
  g.xs = xs;
  g.spo = scale_row_bytes((N >> 1) >> 5);
  g.e = e;
  g.N = N;
  g.K = K;
  g.alpha = alpha;
  g.limit = limit;
  g.F = N >> 1;
  const int KB = K >> 5;
  g.KB = KB;
  g.C = (KB + kChunkBlocks - 1) / kChunkBlocks;             // chunks of 4 blocks
  const int wlast = KB - (g.C - 1) * kChunkBlocks;          // blocks in the last chunk
  g.klast = K - (g.C - 1) * kGmChunkK;                      // k in the last chunk
  g.tid = (int)threadIdx.x;
  const int lane = g.tid & 63, wave = g.tid >> 6;
  g.lr = lane & 15;
  g.lg = lane >> 4;
  g.row0 = row0;

  // weight rows of the wavefront's tiles (first row, rows that exist). A workgroup covers 128
  // h columns (SwiGLU: each wavefront's gate tiles [0, WT/2) and the matching up tiles) or 384
  // rows (plain)
  constexpr int kGmWT = MX8 ? mx_wt(ACT) : gemm_wt(ACT);
  constexpr int kWaves = MX8 ? kMxWaves : kGmWaves;
#pragma unroll
  for (int t = 0; t < kGmWT; ++t) {
    if (swiglu) {
      constexpr int half = kGmWT / 2;
      const int jb = bxi * 128 + wave * 16 * half + 16 * (t % half);
      g.tile_base[t] = (t < half) ? jb : g.F + jb;
      g.rows_in[t] = min(16, g.F - jb);
    } else {
      g.tile_base[t] = bxi * (kWaves * kGmWT * 16) + (wave * kGmWT + t) * 16;
      g.rows_in[t] = min(16, N - g.tile_base[t]);
    }
  }
  static_assert(!swiglu || kWaves * kGmWT * 8 == 128, "128 h columns per workgroup");
  static_assert(swiglu || kWaves * kGmWT * 16 == 384, "384 rows per workgroup");

  // buffer resources: this expert's nibbles and scales, and the activation rows
  const size_t ebase = (size_t)e * N * KB;   // first block of this expert (chunked layout)
  const int SP = scale_row_bytes(KB);        // scale row pitch (padding reads as 0)
  g.spa = SP;                                // MXFP8 activation scale rows use the same pitch
  g.rq = make_rsrc(q + 16 * ebase, (uint32_t)N * KB * 16);
  g.rs = make_rsrc(s + (size_t)e * N * SP, (uint32_t)N * SP);   // SP / 16 groups of N rows
  g.ra = make_rsrc(a, (uint32_t)a_rows * K * (MX8 ? 1 : 2));
  g.ras = make_rsrc(a_scale, MX8 ? (uint32_t)a_rows * SP : 0u);

  // per-lane offsets of the lane's block in a full chunk and in the (narrower) last chunk
#pragma unroll
  for (int t = 0; t < kGmWT; ++t) {
    const uint32_t n = (uint32_t)(g.tile_base[t] + g.lr);
    const bool ok = g.lr < g.rows_in[t];
    g.so[t] = ok ? n * 16 + g.lg : kOOB;   // the row's 16 bytes in a scale group
    g.sg[t] = ok ? n * 16 : kOOB;
    g.wo[t] = ok ? (n * kChunkBlocks + g.lg) * 16 : kOOB;
    g.wol[t] = (ok && g.lg < wlast) ? (n * wlast + g.lg) * 16 : kOOB;
  }

  for (int p0 = 0; p0 < cnt; p0 += kGmTT * 16) {
    g.p0 = p0;
    g.live = min(kGmTT * 16, cnt - p0);
    if constexpr (MX8) {
      switch ((g.live + 15) >> 4) {
        case 1: gemm_pass_mx8<ACT, 1>(g, xs); break;
        case 2: gemm_pass_mx8<ACT, 2>(g, xs); break;
        case 3: gemm_pass_mx8<ACT, 3>(g, xs); break;
        case 4: gemm_pass_mx8<ACT, 4>(g, xs); break;
        case 5: gemm_pass_mx8<ACT, 5>(g, xs); break;
        case 6: gemm_pass_mx8<ACT, 6>(g, xs); break;
        case 7: gemm_pass_mx8<ACT, 7>(g, xs); break;
        default: gemm_pass_mx8<ACT, 8>(g, xs); break;
      }
    } else {
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
}

// Grid and launch of either variant: x = weight-row slices of 128 (SwiGLU) or 384 rows,
// y = expert slots (live experts in id order; slots past the live ones exit at once).
template <bool MX8>
int gemm_launch(const void* a, const uint8_t* a_scale, const int32_t* a_row, int64_t a_rows,
                const mx4_experts* w, const int32_t* counts, const int32_t* basep, int tile_m,
                int64_t mpad_max, int act, float alpha, float limit, void* out,
                uint8_t* out_scale, hipStream_t stream) {
  // buffer resources address at most 2 GB: one expert's weights and the activation matrix
  if ((int64_t)w->N * w->K / 2 >= (1LL << 31) ||
      a_rows * w->K * (MX8 ? 1 : 2) >= (1LL << 31) ||
      a_rows * scale_row_bytes(w->K / 32) >= (1LL << 31))
    return MOE_ESHAPE;
  const int64_t rows_per_wg = 16 * kGmWaves * gemm_wt(MOE_ACT_NONE);
  const int64_t bx = (act != MOE_ACT_NONE) ? (w->N / 2 + 127) / 128
                                            : (w->N + rows_per_wg - 1) / rows_per_wg;
  int64_t slots = mpad_max / tile_m;
  if (slots > w->E) slots = w->E;
  // > 64 KB of dynamic LDS must be opted into, once per kernel and device, at the largest size
  static bool lds_attr_set[kMaxDevices] = {};
  const int lds_max = gemm_lds_bytes(MX8);
  const int dslot = device_slot();
  if (dslot < 0 || !lds_attr_set[dslot]) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<MOE_ACT_NONE, MX8>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds_max) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<MOE_ACT_SWIGLU_OAI, MX8>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds_max) != hipSuccess)
      return MOE_ELAUNCH;
    if (MX8 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<MOE_ACT_SWIGLU_OAI_MX8, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds_max) != hipSuccess)
      return MOE_ELAUNCH;
    if (dslot >= 0) lds_attr_set[dslot] = true;
  }
  const int lds = gemm_lds_bytes(MX8);
  // a 1-D grid of tiles (weight-row slice bx, expert slot), ordered per XCD in the kernel:
  // whole experts per XCD (E <= 64: positions of ceil(slots / 8) experts), else a contiguous
  // share of the tiles
  const int64_t per_xcd = gemm_balanced(w->E, MX8) ? (slots + kXcds - 1) / kXcds * bx
                                                   : (bx * slots + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(per_xcd * kXcds)), block(gemm_threads(MX8));
  if (act == MOE_ACT_SWIGLU_OAI)
    launch(gemm_kernel<MOE_ACT_SWIGLU_OAI, MX8>, grid, block, lds, stream, a, a_scale,
           (int)a_rows, a_row, w->q, w->s, w->bias, counts, basep, w->E, w->N, w->K, alpha,
           limit, out, out_scale, (int)bx, (int)slots, (int)per_xcd);
  else if (act == MOE_ACT_NONE)
    launch(gemm_kernel<MOE_ACT_NONE, MX8>, grid, block, lds, stream, a, a_scale, (int)a_rows,
           a_row, w->q, w->s, w->bias, counts, basep, w->E, w->N, w->K, alpha, limit, out,
           out_scale, (int)bx, (int)slots, (int)per_xcd);
  else if constexpr (MX8)
    launch(gemm_kernel<MOE_ACT_SWIGLU_OAI_MX8, true>, grid, block, lds, stream, a, a_scale,
           (int)a_rows, a_row, w->q, w->s, w->bias, counts, basep, w->E, w->N, w->K, alpha,
           limit, out, out_scale, (int)bx, (int)slots, (int)per_xcd);
  else
    return MOE_EINVAL;
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

}  // namespace moe

int moe_launch_gemm(const uint16_t* a, const int32_t* a_row, int64_t a_rows, const mx4_experts* w,
                    const int32_t* counts, const int32_t* basep, int tile_m, int64_t mpad_max,
                    int act, float alpha, float limit, void* out, hipStream_t stream) {
  return moe::gemm_launch<false>(a, nullptr, a_row, a_rows, w, counts, basep, tile_m, mpad_max,
                                 act, alpha, limit, out, nullptr, stream);
}

int moe_launch_gemm_mx8(const uint8_t* aq, const uint8_t* as, const int32_t* a_row,
                        int64_t a_rows, const mx4_experts* w, const int32_t* counts,
                        const int32_t* basep, int tile_m, int64_t mpad_max, int act, float alpha,
                        float limit, void* out, uint8_t* out_scale, hipStream_t stream) {
  return moe::gemm_launch<true>(aq, as, a_row, a_rows, w, counts, basep, tile_m, mpad_max, act,
                                alpha, limit, out, out_scale, stream);
}
