// moe_route_topk: top-k expert selection and softmax routing weights, one wavefront per token.
//
// Each token picks its k largest router logits, in descending order with equal logits ordered by
// ascending expert id; its routing weights are the softmax over the k selected logits, computed
// in double and rounded to f32 (gpt-oss router). The chain's per-token expert ids and k = 4 at
// gpt-oss shape come from PR #3579 "dasLLAMA gpt-oss arc" (fused MoE expert chain commit) and
// PR #3558 (section "gpt-oss: mx4 kernels to the lab-winning shape").
#include "common.hpp"

namespace moe {

constexpr int kRouteThreads = 256;                   // 4 tokens per workgroup
constexpr int kRoutePerLane = MOE_MAX_E / kWave;     // logits held per lane

// better(a, b): a ranks before b (larger value; ties -> lower id). -0.0 == +0.0 as floats.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return (va > vb) || (va == vb && ia < ib);
}

__global__ void __launch_bounds__(kRouteThreads)
route_topk_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                  int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = (int)(threadIdx.x & 63);
  const int64_t t = (int64_t)blockIdx.x * (kRouteThreads / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront leaves together
  const float* row = logits + t * (int64_t)E;

  float v[kRoutePerLane];
#pragma unroll
  for (int j = 0; j < kRoutePerLane; ++j) {
    const int e = j * kWave + lane;
    v[j] = (e < E) ? row[e] : 0.0f;
  }
  uint32_t taken = 0;                 // bit j: expert j*64+lane already chosen (or absent)
#pragma unroll
  for (int j = 0; j < kRoutePerLane; ++j)
    if (j * kWave + lane >= E) taken |= 1u << j;

  float sel_v[MOE_MAX_K];
  int sel_id[MOE_MAX_K];
  for (int s = 0; s < k; ++s) {
    // this lane's best remaining candidate
    float bv = 0.0f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kRoutePerLane; ++j) {
      const int e = j * kWave + lane;
      if (!(taken & (1u << j)) && (bi == 0x7FFFFFFF || ranks_before(v[j], e, bv, bi))) {
        bv = v[j];
        bi = e;
      }
    }
    // wavefront arg-best (lanes without a candidate carry id INT_MAX and never win)
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m);
      const int oi = __shfl_xor(bi, m);
      if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || ranks_before(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
      }
    }
    sel_v[s] = bv;
    sel_id[s] = bi;
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
  }

  if (lane == 0) {
    const double l0 = (double)sel_v[0];
    double num[MOE_MAX_K];
    double den = 0.0;
    for (int s = 0; s < k; ++s) {
      num[s] = exp((double)sel_v[s] - l0);
      den += num[s];
    }
    for (int s = 0; s < k; ++s) {
      ids[t * k + s] = sel_id[s];
      w[t * k + s] = (float)(num[s] / den);
    }
  }
}

}  // namespace moe

extern "C" int moe_route_topk(const float* logits, int64_t T, int E, int k, int32_t* ids,
                              float* w, void* stream) {
  if (!logits || !ids || !w || T < 1 || E < 1 || k < 1 || k > E || k > MOE_MAX_K)
    return MOE_EINVAL;
  if (E > MOE_MAX_E) return MOE_ESHAPE;
  const int per_block = moe::kRouteThreads / moe::kWave;
  const int64_t blocks = (T + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFF) return MOE_ESHAPE;
  hipLaunchKernelGGL(moe::route_topk_kernel, dim3((unsigned)blocks), dim3(moe::kRouteThreads), 0,
                     (hipStream_t)stream, logits, T, E, k, ids, w);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
