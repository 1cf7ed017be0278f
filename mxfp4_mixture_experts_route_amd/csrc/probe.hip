// Attained-peak probes, for measurement only: a plain streaming read of a buffer (the HBM rate
// a simple kernel attains at a given size) and a loop of bf16 MFMAs (the matrix-core rate a
// kernel attains with nothing else to do). They put the roofline fractions of the chain's
// kernels beside what the chip delivers in practice, not only beside its published peaks.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;    // 16-byte loads in flight per lane

// Every byte of src read once (16 bytes per lane per load, nontemporal, 8 loads in flight,
// grid-stride in units of 8 whole-grid strides); the xor of all words is written only if it
// equals a value no real input produces by chance (so the loads cannot be dropped, and nothing
// is written). Of the plain read shapes tried (grid-stride or a contiguous slab per workgroup,
// 8 or 16 loads in flight, with and without the nontemporal hint, 256 to 4096 workgroups),
// this one was the fastest or within 1 % of it at every size.
__global__ void __launch_bounds__(kProbeThreads)
probe_read_kernel(const u32x4_t* __restrict__ src, int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// iters x 4 independent v_mfma_f32_32x32x16_bf16 per wavefront (4 accumulator chains of 16
// registers, so the matrix core never waits for a result; the compiler keeps the loop free of
// accumulator copies in this form, which it does not for 16x16x32 chains); 4 wavefronts per
// workgroup, one per SIMD.
__global__ void __launch_bounds__(kProbeThreads)
probe_mfma_kernel(int iters, float* __restrict__ sink) {
  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  const float t = (float)(threadIdx.x & 63) * 1e-3f;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(t + (float)i);
    b[i] = (__bf16)(1.0f - t * (float)i);
  }
  f32x16_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc[j] = f32x16_t{};
    acc[j][0] = t;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) s += acc[j][q];
  if (s == 1234.5f) sink[0] = s;
}

}  // namespace moe

extern "C" int moe_probe_read(const void* src, int64_t bytes, uint32_t* sink, int workgroups,
                              void* stream) {
  if (!src || !sink || bytes < 16 || workgroups < 1) return MOE_EINVAL;
  if ((((uintptr_t)src) & 15) || (bytes & 15)) return MOE_EALIGN;
  moe::launch(moe::probe_read_kernel, dim3((unsigned)workgroups), dim3(moe::kProbeThreads), 0,
              (hipStream_t)stream, reinterpret_cast<const moe::u32x4_t*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

extern "C" int moe_probe_mfma_bf16(int workgroups, int iters, float* sink, void* stream) {
  if (!sink || workgroups < 1 || iters < 1) return MOE_EINVAL;
  moe::launch(moe::probe_mfma_kernel, dim3((unsigned)workgroups), dim3(moe::kProbeThreads), 0,
              (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
