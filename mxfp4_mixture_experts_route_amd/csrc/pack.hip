// mx4_pack_experts: checkpoint (row-major) MXFP4 layout -> chunked layout read by the projections.
//
// A pure byte permutation, run once when weights are loaded: one thread per 16-byte MX block,
// reading the source in order (coalesced) and writing the block to its chunked position and its
// scale byte to its scale group (16 blocks of one row; all rows of a group together). The chunked layout makes each wavefront load of the projection kernels one
// contiguous 1 KB run and keeps all workgroups of a launch inside a compact window of memory.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kPackThreads = 256;

__global__ void __launch_bounds__(kPackThreads)
pack_kernel(const uint8_t* __restrict__ q_src, const uint8_t* __restrict__ s_src, int E, int N,
            int KB, uint8_t* __restrict__ q_dst, uint8_t* __restrict__ s_dst) {
  const size_t total = (size_t)E * N * KB;
  const int G = scale_row_bytes(KB) / 16;   // scale groups per row
  for (size_t i = (size_t)blockIdx.x * kPackThreads + threadIdx.x; i < total;
       i += (size_t)gridDim.x * kPackThreads) {
    const int kb = (int)(i % KB);
    const size_t row = i / KB;
    const int n = (int)(row % N);
    const int e = (int)(row / N);
    const size_t d = chunked_block(e, n, kb, N, KB);
    *reinterpret_cast<uint4*>(q_dst + 16 * d) = *reinterpret_cast<const uint4*>(q_src + 16 * i);
    uint8_t* grp = s_dst + 16 * (((size_t)e * G + kb / 16) * N + n);
    grp[kb % 16] = s_src[i];
    if (kb == KB - 1)
      for (int p = kb % 16 + 1; p < 16; ++p) grp[p] = 0;   // padding of the last group
  }
}

}  // namespace moe

extern "C" int mx4_pack_experts(const uint8_t* q_src, const uint8_t* s_src, int E, int N, int K,
                                uint8_t* q_dst, uint8_t* s_dst, void* stream) {
  if (!q_src || !s_src || !q_dst || !s_dst || E < 1 || N < 1) return MOE_EINVAL;
  if (K < 32 || (K % 32) != 0) return MOE_ESHAPE;
  if ((((uintptr_t)q_src) & 15) || (((uintptr_t)q_dst) & 15) || (((uintptr_t)s_dst) & 15))
    return MOE_EALIGN;
  const size_t total = (size_t)E * N * (K / 32);
  size_t blocks = (total + moe::kPackThreads - 1) / moe::kPackThreads;
  if (blocks > 65536) blocks = 65536;
  moe::launch(moe::pack_kernel, dim3((unsigned)blocks), dim3(moe::kPackThreads), 0,
                     (hipStream_t)stream, q_src, s_src, E, N, K / 32, q_dst, s_dst);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
