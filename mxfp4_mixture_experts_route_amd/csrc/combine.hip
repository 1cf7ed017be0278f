// moe_combine: router-weighted sum of each token's expert rows, in slot order.
//
// PR #3579 "dasLLAMA gpt-oss arc", PR body section "Fused MoE expert chain" and the fused chain
// commit: the second stage takes every routed expert's down row (bias included) and forms the
// routing-weighted sum in slot order. y[t][n] = sum_s w[t][s] * d[pos[t][s]][n], fp32, s = 0..k-1.
// One thread per 4 consecutive outputs; each d row segment is read with 16-byte loads.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kCombineThreads = 256;

__global__ void __launch_bounds__(kCombineThreads)
combine_kernel(const float* __restrict__ d, int64_t d_rows, const int32_t* __restrict__ pos,
               const float* __restrict__ w, int64_t T, int k, int D, float* __restrict__ y,
               int vec) {
  const int quads = (D + 3) >> 2;
  const int64_t gid = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  if (gid >= T * (int64_t)quads) return;
  const int64_t t = gid / quads;
  const int n0 = (int)(gid - t * quads) * 4;
  const bool full = vec && (n0 + 4 <= D);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < k; ++s) {
    const int64_t r = pos[t * k + s];
    const float ws = w[t * k + s];
    if ((uint64_t)r >= (uint64_t)d_rows) continue;  // precondition breach: skip, never fault
    const float* src = d + r * (int64_t)D + n0;
    if (full) {
      const float4 v = *reinterpret_cast<const float4*>(src);
      acc[0] = fmaf(ws, v.x, acc[0]);
      acc[1] = fmaf(ws, v.y, acc[1]);
      acc[2] = fmaf(ws, v.z, acc[2]);
      acc[3] = fmaf(ws, v.w, acc[3]);
    } else {
      for (int i = 0; i < 4 && n0 + i < D; ++i) acc[i] = fmaf(ws, src[i], acc[i]);
    }
  }
  float* dst = y + t * (int64_t)D + n0;
  if (full) {
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
    for (int i = 0; i < 4 && n0 + i < D; ++i) dst[i] = acc[i];
  }
}

}  // namespace moe

extern "C" int moe_combine(const float* d, int64_t d_rows, const int32_t* pos, const float* w,
                           int64_t T, int k, int D, float* y, void* stream) {
  if (!d || !pos || !w || !y || T < 1 || k < 1 || k > MOE_MAX_K || D < 1 || d_rows < 1)
    return MOE_EINVAL;
  if ((((uintptr_t)d) & 3) || (((uintptr_t)y) & 3)) return MOE_EALIGN;
  const int64_t quads = (D + 3) / 4;
  const int64_t blocks = (T * quads + moe::kCombineThreads - 1) / moe::kCombineThreads;
  if (blocks > 0x7FFFFFFF) return MOE_ESHAPE;
  // 16-byte vector access when every row starts 16-byte aligned; otherwise the scalar path
  const int vec = ((D & 3) == 0) && !(((uintptr_t)d) & 15) && !(((uintptr_t)y) & 15);
  moe::launch(moe::combine_kernel, dim3((unsigned)blocks), dim3(moe::kCombineThreads), 0,
                     (hipStream_t)stream, d, d_rows, pos, w, T, k, D, y, vec);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
