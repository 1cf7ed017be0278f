// moe_route_topk: top-k expert selection and softmax routing weights, one wavefront per token.
//
// Each token picks its k largest router logits, in descending order with equal logits ordered by
// ascending expert id; its routing weights are the softmax over the k selected logits, computed
// in double and rounded to f32 (gpt-oss router). The chain's per-token expert ids and k = 4 at
// gpt-oss shape come from PR #3579 "dasLLAMA gpt-oss arc" (fused MoE expert chain commit) and
// PR #3558 (section "gpt-oss: mx4 kernels to the lab-winning shape").
#include "route_core.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kRouteThreads = 256;                   // 4 tokens per workgroup

__global__ void __launch_bounds__(kRouteThreads)
route_topk_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                  int32_t* __restrict__ ids, float* __restrict__ w) {
  const int64_t t = (int64_t)blockIdx.x * (kRouteThreads / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront leaves together
  int my_id;
  float my_v;
  wave_topk(logits + t * (int64_t)E, E, k, my_id, my_v);
  write_topk(my_id, my_v, k, ids + t * k, w + t * k);
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
  moe::launch(moe::route_topk_kernel, dim3((unsigned)blocks), dim3(moe::kRouteThreads), 0,
                     (hipStream_t)stream, logits, T, E, k, ids, w);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
