// Device-side helpers shared by the kernels of the routed MXFP4 MoE chain (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_mx4.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// operand formats of v_mfma_scale_f32_*_f8f6f4 (the cbsz / blgp fields)
constexpr int kMfmaFmtFp8 = 0;   // E4M3
constexpr int kMfmaFmtFp4 = 4;   // E2M1

constexpr int kWave = 64;
constexpr int kChunkBlocks = 4;   // MX blocks per chunk of the chunked weight layout

// Raw buffer resource over `bytes` bytes at p (gfx9 family: dword3 = 0x00020000, stride 0).
// Buffer loads whose offset lands at or past `bytes` return zeros instead of touching memory,
// which is how the kernels below handle tails and invalid lanes without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOOB = 0x80000000u;   // a buffer offset past every resource: loads give zero

__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  u32x4_t out;
  __builtin_memcpy(&out, &v, sizeof(out));
  return out;
}

// The same with the nontemporal hint (weights streamed once: they should not displace what
// the caches hold for other wavefronts; measured 1.5-2 us faster on the one-launch decode layer)
__device__ __forceinline__ u32x4_t buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);
  u32x4_t out;
  __builtin_memcpy(&out, &v, sizeof(out));
  return out;
}

__device__ __forceinline__ uint32_t buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

// Keeps the memory operations before and after it in program order: an empty asm statement
// that clobbers memory stops IR passes from sinking or hoisting loads across it, and the
// scheduling barrier stops the machine scheduler. Vector loads complete in issue order, so the
// compiler's own wait counts depend on that order.
__device__ __forceinline__ void issue_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most n (<= 63) vector-memory
// operations of this wavefront are outstanding, and for nothing else.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Block number of block kb of row n of expert e in the chunked MXFP4 layout: the expert's K is
// cut into chunks of 4 blocks stored one after another, all N rows of a chunk together (the
// last chunk may be narrower). Its 16 nibble bytes start at byte 16 * number.
__host__ __device__ __forceinline__ size_t chunked_block(int e, int n, int kb, int N, int KB) {
  const int c = kb / kChunkBlocks;
  const int w = (KB - c * kChunkBlocks) < kChunkBlocks ? (KB - c * kChunkBlocks) : kChunkBlocks;
  return (size_t)e * N * KB + (size_t)c * N * kChunkBlocks + (size_t)n * w + (kb % kChunkBlocks);
}

// Bytes per scale row of the chunked layout: the row's KB scale bytes padded to 16.
__host__ __device__ __forceinline__ int scale_row_bytes(int KB) { return (KB + 15) & ~15; }

// Four bias seeds of a 16-row MFMA tile, through the scalar cache: lane (lr, lg) gets rows
// 4lg..4lg+3 of rows lo[0..7] (tile rows 0-7) and hi[0..7] (tile rows 8-15). lo and hi must be the
// same on every lane (they are made so). A scalar load is not counted by the vector-memory
// counter, so a wavefront that waits for its weight chunks in issue order never waits for its
// seeds behind them (a vector load of the seeds, issued after the routing, arrives behind the
// whole weight flood of the launch).
__device__ __forceinline__ void scalar_seed16(const float* lo, const float* hi, float (&b4)[4]) {
  typedef const __attribute__((address_space(4))) float* cfp;
  const cfp cl = (cfp)lo, ch = (cfp)hi;
  float g[8], u[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    g[i] = cl[i];
    u[i] = ch[i];
  }
  const int lg = (int)(threadIdx.x & 63) >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    b4[i] = lg == 0 ? g[i] : lg == 1 ? g[4 + i] : lg == 2 ? u[i] : u[4 + i];
}

// Scale operand of v_cvt_scalef32_* for an e8m0 byte e: the byte in the fp32 exponent field.
// The instruction reads only that field and decodes it as e8m0 itself: 2^(e-127), with e = 0
// giving 2^-127 (subnormal results kept) and e = 255 giving NaN; checked on gfx950 against the
// explicit decode for every (scale byte, code byte) pair, and end to end by the one-hot sweep.
__device__ __forceinline__ float e8m0_scale_operand(uint32_t e) { return __uint_as_float(e << 23); }

// 8 e2m1 codes (one dword of an MX block: elements 8t..8t+7, element 2b in the low nibble of
// byte b) -> 8 bf16 scaled by the block's e8m0 scale operand; exact.
__device__ __forceinline__ bf16x8_t dequant8(uint32_t w8, float scale) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w8, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w8, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w8, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w8, scale, 3);
  return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// float -> bf16 bit pattern, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Reinterpret a dword as two bf16 (element 0 = low half). Take the dword as a scalar first:
// clang (ROCm 7.2) miscompiles __builtin_bit_cast applied directly to an ext-vector element,
// reading element 0 whatever the index.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) {
  bf16x2_t r;
  __builtin_memcpy(&r, &u, sizeof(r));
  return r;
}

// E4M3 byte of a finite fp32 value t with |t| < 2^9, round to nearest even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float t) {
  const uint32_t u = __float_as_uint(t);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t mag;
  if (a < 0x3C800000u) {                      // |t| < 2^-6: subnormal step 2^-9
    // |t| * 2^9 < 8 is exact; rintf rounds half to even; 8 lands on 2^-6 = byte 0x08
    mag = (uint32_t)rintf(__uint_as_float(a) * 512.0f);
  } else {
    // keep 3 mantissa bits, rounding half to even (a carry into the exponent is a correct
    // round up to the next binade)
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    const int ex = (int)(r >> 23) - 127;      // >= -6
    const uint32_t m3 = (r >> 20) & 7u;
    mag = (ex > 8 || (ex == 8 && m3 == 7u)) ? 0x7Eu : ((uint32_t)(ex + 7) << 3) | m3;
  }
  return sign | mag;
}

// MXFP8 scale byte of a 32-value block whose largest magnitude, as a bf16 pattern with the sign
// cleared, is amax (OCP MX: exponent of the maximum minus 8, clamped at e8m0 byte 0), and the
// exact factor 2^-X that scales the block's values onto the E4M3 grid.
__device__ __forceinline__ uint32_t mx8_scale_byte(uint32_t amax) {
  const int ea = (int)(amax >> 7);
  return (uint32_t)max(ea - 8, 0);
}
__device__ __forceinline__ float mx8_inv_scale(uint32_t sbyte) {
  return __uint_as_float((254u - sbyte) << 23);   // 2^(127 - sbyte), a normal float
}

// Clamped SwiGLU-OAI of one (gate, up) pair: gc = min(gate, limit), uc = clamp(up, +-limit),
// gc * sigmoid(alpha*gc) * (uc + 1). The sigmoid is evaluated on the side where the exponential
// cannot overflow (e = exp(-|z|) <= 1). exp(-|z|) = 2^(-|z| log2 e) and 1 / (1 + e) use the
// hardware's exp2 and reciprocal (about 1 ulp each, far below the bf16 rounding of h); the
// accurate library exp and IEEE division cost ~40 VALU ops per value in epilogues that run
// while HBM idles. The hardware exp2 returns 0 below the normal range (2^-126), which for very
// negative gates (|z| beyond ~87) would zero an h that bf16 still represents (its smallest
// magnitude is 2^-133): there the exponent is taken 64 higher, exactly (|z| log2 e >= 64 has
// no bits below 2^-17), and the product is scaled back by 2^-64 at the end.
__device__ __forceinline__ float swiglu_oai(float gate, float up, float alpha, float limit) {
  const float gc = fminf(gate, limit);
  const float uc = fminf(fmaxf(up, -limit), limit);
  const float z = alpha * gc;
  const float x = -fabsf(z) * 1.44269504088896341f;
  const bool tiny = x < -64.0f;                                   // e < 2^-64
  const float es = __builtin_amdgcn_exp2f(tiny ? x + 64.0f : x);  // e, times 2^64 when tiny
  const float r = __builtin_amdgcn_rcpf(1.0f + (tiny ? 0.0f : es));
  const float h = gc * ((z >= 0.0f) ? r : es * r) * (uc + 1.0f);
  return (tiny && z < 0.0f) ? h * 0x1p-64f : h;
}

// Sum over the 16 lanes of each DPP row (lanes 16r..16r+15); every lane gets the row's sum.
// Fixed butterfly order, so the result is deterministic.
__device__ __forceinline__ float row16_sum(float v) {
  v += __shfl_xor(v, 8, 16);
  v += __shfl_xor(v, 4, 16);
  v += __shfl_xor(v, 2, 16);
  v += __shfl_xor(v, 1, 16);
  return v;
}

// Index of the slot-th expert with a non-zero count, or -1; computed by every thread of the
// block (the block's threads scan counts[] together). Needs blockDim.x == 256 and a
// __shared__ int scratch[2].
__device__ __forceinline__ int slot_expert(const int32_t* __restrict__ counts, int E, int slot,
                                           int* scratch) {
  if (threadIdx.x == 0) scratch[0] = -1;
  __syncthreads();
  int seen = 0;
  for (int base = 0; base < E; base += 256) {
    const int e = base + (int)threadIdx.x;
    const bool live = (e < E) && (counts[e] > 0);
    // block-wide exclusive rank of this live expert
    const uint64_t ballot = __ballot(live);
    const int lane = (int)(threadIdx.x & 63);
    const int wave = (int)(threadIdx.x >> 6);
    const int in_wave = __popcll(ballot & ((lane ? (~0ull >> (64 - lane)) : 0ull)));
    __shared__ int wave_tot[4];
    if (lane == 0) wave_tot[wave] = __popcll(ballot);
    __syncthreads();
    int before = seen;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    if (live && before + in_wave == slot) scratch[0] = e;
    seen += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    __syncthreads();
  }
  return scratch[0];
}

}  // namespace moe
