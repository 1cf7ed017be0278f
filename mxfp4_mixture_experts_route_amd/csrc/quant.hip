// mx8_quantize: bf16 rows -> MXFP8 rows (E4M3 elements, one e8m0 scale per 32 values), the
// activation format of the projections on the MX-scaled MFMA.
//
// The pages quantize only the weights; the format and the conversion follow the OCP 8-bit
// floating point spec (E4M3: bias 7, 3 mantissa bits, subnormal step 2^-9, largest finite 448,
// no infinities) and the OCP Microscaling v1.0 spec (a block's shared exponent is the exponent
// of its largest magnitude minus that of the element format's largest normal; elements are
// rounded to nearest even and clamped to the largest finite value).
//
// One lane per 32-value block: it loads the block's 64 bytes, takes the largest magnitude as
// an integer maximum of the bf16 bit patterns with the sign cleared (for non-negative floats
// the integer order is the float order), reads the exponent field off it, and converts the 32
// scaled values with integer rounding. Adjacent lanes take adjacent blocks of a row, so each
// wavefront reads 4 KB and writes 2 KB of contiguous memory. Every step is exact: v / 2^X is a
// power-of-two scaling of a bf16 value, so the result is the same as rounding the exact
// quotient.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

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

__global__ void __launch_bounds__(256)
mx8_quantize_kernel(const uint16_t* __restrict__ a, const int32_t* __restrict__ live,
                    int64_t rows, int K, uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int KB = K >> 5;
  const int SP = scale_row_bytes(KB);
  const int64_t unit = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (unit >= rows * KB) return;
  const int64_t r = unit / KB;
  const int b = (int)(unit - r * KB);
  if (live && live[r] < 0) return;
  const uint4* src = reinterpret_cast<const uint4*>(a + r * K + (int64_t)b * 32);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    w[4 * i + 0] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
  uint32_t amax = 0;   // largest |value| as a bf16 pattern (sign cleared)
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    amax = max(amax, w[i] & 0x7FFFu);
    amax = max(amax, (w[i] >> 16) & 0x7FFFu);
  }
  // exponent field Ea of the largest magnitude: floor(log2 m) = Ea - 127 for a normal m, so
  // the scale byte X + 127 = Ea - 8, clamped at 0 (a zero or subnormal m has Ea = 0)
  const int ea = (int)(amax >> 7);
  const uint32_t sbyte = (uint32_t)max(ea - 8, 0);
  const float inv = __uint_as_float((254u - sbyte) << 23);   // 2^(127 - sbyte) = 2^-X, exact
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t pk = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * i + j;   // element e of the block: low half of w[e/2] when e is even
      const uint32_t bits = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
      pk |= e4m3_rne_sat(bf16_bits_to_f32(bits) * inv) << (8 * j);
    }
    out[i] = pk;
  }
  uint4* dst = reinterpret_cast<uint4*>(q + r * K + (int64_t)b * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  uint8_t* srow = s + r * SP;
  srow[b] = (uint8_t)sbyte;
  if (b == KB - 1)
    for (int p = KB; p < SP; ++p) srow[p] = 0;   // the row's padding
}

}  // namespace moe

extern "C" int mx8_quantize(const uint16_t* a, const int32_t* live, int64_t rows, int K,
                            uint8_t* q, uint8_t* s, void* stream) {
  if (!a || !q || !s || rows < 1) return MOE_EINVAL;
  if (K < 32 || (K % 32) != 0 || rows * (int64_t)K >= (1LL << 31)) return MOE_ESHAPE;
  if ((((uintptr_t)a) & 15) || (((uintptr_t)q) & 15) || (((uintptr_t)s) & 15)) return MOE_EALIGN;
  const int64_t units = rows * (K / 32);
  moe::launch(moe::mx8_quantize_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0,
              (hipStream_t)stream, a, live, rows, K, q, s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
