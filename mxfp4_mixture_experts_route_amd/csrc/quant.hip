// mx8_quantize: bf16 rows -> MXFP8 rows (E4M3 elements, one e8m0 scale per 32 values), the
// activation format of the projections on the MX-scaled MFMA.
//
// The pages quantize only the weights; the format and the conversion follow the OCP 8-bit
// floating point spec (E4M3: bias 7, 3 mantissa bits, subnormal step 2^-9, largest finite 448,
// no infinities) and the OCP Microscaling v1.0 spec (a block's shared exponent is the exponent
// of its largest magnitude minus that of the element format's largest normal; elements are
// rounded to nearest even and clamped to the largest finite value).
//
// Four lanes per 32-value block: each loads 16 bytes, the group takes the largest magnitude as
// an integer maximum of the bf16 bit patterns with the sign cleared (for non-negative floats
// the integer order is the float order), reads the exponent field off it, and converts its 8
// scaled values with integer rounding. Every step is exact: v / 2^X is a power-of-two scaling
// of a bf16 value, so the result is the same as rounding the exact quotient.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// Four lanes per 32-value block, 8 values (16 bytes) each: a wavefront covers 16 consecutive
// blocks, i.e. 1 KB of bf16 read and 512 bytes of E4M3 written, contiguous across its lanes.
__global__ void __launch_bounds__(256)
mx8_quantize_kernel(const uint16_t* __restrict__ a, const int32_t* __restrict__ live,
                    int64_t rows, int K, uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int KB = K >> 5;
  const int SP = scale_row_bytes(KB);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t unit = gid >> 2;            // block (row-major over rows x KB)
  const int part = (int)(gid & 3);          // values 8*part .. 8*part+7 of the block
  // whole groups of 4 lanes leave together, so the group's shuffles below see live partners
  const bool in_range = unit < rows * KB;
  const int64_t r = in_range ? unit / KB : 0;
  const int b = in_range ? (int)(unit - r * KB) : 0;
  const bool active = in_range && !(live && live[r] < 0);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (active) v = *reinterpret_cast<const uint4*>(a + r * K + (int64_t)b * 32 + part * 8);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t amax = 0;   // largest |value| as a bf16 pattern (sign cleared)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    amax = max(amax, w[i] & 0x7FFFu);
    amax = max(amax, (w[i] >> 16) & 0x7FFFu);
  }
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1, 4));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2, 4));
  if (!active) return;
  // exponent field Ea of the largest magnitude: floor(log2 m) = Ea - 127 for a normal m, so
  // the scale byte X + 127 = Ea - 8, clamped at 0 (a zero or subnormal m has Ea = 0)
  const uint32_t sbyte = mx8_scale_byte(amax);
  const float inv = mx8_inv_scale(sbyte);   // 2^(127 - sbyte) = 2^-X, exact
  uint32_t out[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t pk = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * i + j;   // value e of the lane: low half of w[e/2] when e is even
      const uint32_t bits = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
      pk |= e4m3_rne_sat(bf16_bits_to_f32(bits) * inv) << (8 * j);
    }
    out[i] = pk;
  }
  *reinterpret_cast<uint2*>(q + r * K + (int64_t)b * 32 + part * 8) = make_uint2(out[0], out[1]);
  uint8_t* srow = s + r * SP;
  if (part == 0) srow[b] = (uint8_t)sbyte;
  if (part == 1 && b == KB - 1)
    for (int p = KB; p < SP; ++p) srow[p] = 0;   // the row's padding
}

}  // namespace moe

extern "C" int mx8_quantize(const uint16_t* a, const int32_t* live, int64_t rows, int K,
                            uint8_t* q, uint8_t* s, void* stream) {
  if (!a || !q || !s || rows < 1) return MOE_EINVAL;
  if (K < 32 || (K % 32) != 0 || rows * (int64_t)K >= (1LL << 31)) return MOE_ESHAPE;
  if ((((uintptr_t)a) & 15) || (((uintptr_t)q) & 15) || (((uintptr_t)s) & 15)) return MOE_EALIGN;
  const int64_t lanes = rows * (K / 32) * 4;
  moe::launch(moe::mx8_quantize_kernel, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0,
              (hipStream_t)stream, a, live, rows, K, q, s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
