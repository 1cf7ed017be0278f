// moe_bucket: CSR of routed rows per expert with padded prefix bases, one workgroup per expert.
//
// PR #3579 "dasLLAMA gpt-oss arc", commit log, Metal fusion-lane commit: the bucket pass gives
// each expert one workgroup, which computes that expert's padded-prefix base itself and publishes
// it, so no separate serial prefix pass (and no extra dispatch or barrier level) is needed; the
// CSR it produces is the same bit for bit. Here every workgroup histograms all T*k ids in LDS,
// sums the padded counts of the experts below its own to get basep[e], then compacts its rows in
// ascending token order with wavefront ballots (an ordered scan, so the result is unique). The
// ids are read kBucketUnroll loads at a time per thread (all in flight before the histogram's
// atomics) and, when T*k fits kBucketStaged ids, kept in LDS for the compaction, which then
// reads no memory.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kBucketThreads = 256;
constexpr int kBucketUnroll = 8;          // id loads in flight per thread
constexpr int kBucketStaged = 12 * 1024;  // ids kept in LDS for the compaction (48 KB), at most

__global__ void __launch_bounds__(kBucketThreads)
bucket_kernel(const int32_t* __restrict__ ids, int64_t T, int k, int E, int tile_m,
              int64_t mpad_max, int32_t* __restrict__ counts, int32_t* __restrict__ basep,
              int32_t* __restrict__ row_tok, int32_t* __restrict__ pos, int staged) {
  extern __shared__ int idl[];   // [T*k] when staged
  __shared__ int hist[MOE_MAX_E];
  __shared__ int red[kBucketThreads / kWave][2];
  __shared__ int wave_tot[kBucketThreads / kWave];
  const int e = (int)blockIdx.x;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t R = T * (int64_t)k;

  for (int i = tid; i < E; i += kBucketThreads) hist[i] = 0;
  __syncthreads();
  for (int64_t i0 = 0; i0 < R; i0 += (int64_t)kBucketThreads * kBucketUnroll) {
    int v[kBucketUnroll];
#pragma unroll
    for (int u = 0; u < kBucketUnroll; ++u) {
      const int64_t i = i0 + u * kBucketThreads + tid;
      v[u] = i < R ? ids[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < kBucketUnroll; ++u) {
      const int64_t i = i0 + u * kBucketThreads + tid;
      if (staged && i < R) idl[i] = v[u];
      if ((unsigned)v[u] < (unsigned)E) atomicAdd(&hist[v[u]], 1);  // ids outside [0,E): ignored
    }
  }
  __syncthreads();

  // basep[e] = sum over e' < e of roundup(cnt[e'], tile_m); total = the same over all experts
  int below = 0, total = 0;
  for (int i = tid; i < E; i += kBucketThreads) {
    const int padded = (hist[i] + tile_m - 1) / tile_m * tile_m;
    total += padded;
    if (i < e) below += padded;
  }
  for (int m = 32; m >= 1; m >>= 1) {
    below += __shfl_xor(below, m);
    total += __shfl_xor(total, m);
  }
  if (lane == 0) {
    red[wave][0] = below;
    red[wave][1] = total;
  }
  __syncthreads();
  below = red[0][0] + red[1][0] + red[2][0] + red[3][0];
  total = red[0][1] + red[1][1] + red[2][1] + red[3][1];
  const int cnt = hist[e];
  const int padded = (cnt + tile_m - 1) / tile_m * tile_m;

  if (tid == 0) {
    counts[e] = cnt;
    basep[e] = below;
    if (e == E - 1) basep[E] = total;
  }

  // ordered compaction: this expert's (t, s) pairs in ascending t
  int running = 0;
  for (int64_t t0 = 0; t0 < T; t0 += kBucketThreads) {
    const int64_t t = t0 + tid;
    int slot = -1;
    if (t < T)
      for (int s = 0; s < k; ++s)
        if ((staged ? idl[t * k + s] : ids[t * k + s]) == e) slot = s;
    const uint64_t ballot = __ballot(slot >= 0);
    const int in_wave = __popcll(ballot & (lane ? (~0ull >> (64 - lane)) : 0ull));
    if (lane == 0) wave_tot[wave] = __popcll(ballot);
    __syncthreads();
    int before = running;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    if (slot >= 0) {
      const int r = below + before + in_wave;
      row_tok[r] = (int32_t)t;
      pos[t * k + slot] = r;
    }
    running += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    __syncthreads();
  }

  // padding rows of this bucket, and a share of the ghost rows past the last bucket
  for (int r = below + cnt + tid; r < below + padded; r += kBucketThreads) row_tok[r] = -1;
  for (int64_t r = (int64_t)total + (int64_t)e * kBucketThreads + tid; r < mpad_max;
       r += (int64_t)E * kBucketThreads)
    row_tok[r] = -1;
}

}  // namespace moe

extern "C" int64_t moe_mpad_max(int64_t T, int k, int E, int tile_m) {
  if (T < 1 || k < 1 || E < 1 || k > E || tile_m < 1) return -1;
  const int64_t R = T * (int64_t)k;
  const int64_t n = R + (R < E ? R : (int64_t)E) * (tile_m - 1);
  return (n + tile_m - 1) / tile_m * tile_m;
}

extern "C" int moe_bucket(const int32_t* ids, int64_t T, int k, int E, int tile_m,
                          int64_t mpad_max, int32_t* counts, int32_t* basep, int32_t* row_tok,
                          int32_t* pos, void* stream) {
  if (!ids || !counts || !basep || !row_tok || !pos || T < 1 || k < 1 || E < 1 || k > E ||
      k > MOE_MAX_K)
    return MOE_EINVAL;
  if (E > MOE_MAX_E || tile_m < 1 || tile_m > MOE_MAX_TILE_M) return MOE_ESHAPE;
  const int64_t need = moe_mpad_max(T, k, E, tile_m);
  if (mpad_max < need || mpad_max > 0x7FFFFFFFLL) return MOE_ESHAPE;
  const int64_t R = T * (int64_t)k;
  const int staged = R <= moe::kBucketStaged ? 1 : 0;
  moe::launch(moe::bucket_kernel, dim3((unsigned)E), dim3(moe::kBucketThreads),
              staged ? (size_t)R * sizeof(int) : 0, (hipStream_t)stream, ids, T, k, E, tile_m,
              mpad_max, counts, basep, row_tok, pos, staged);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
