// Top-k expert selection of one token by one wavefront (shared by moe_route_topk and the fused
// decode layer).
//
// A token picks its k largest router logits, in descending order, equal logits ordered by
// ascending expert id; its routing weights are the softmax over the k selected logits, computed
// in double relative to the largest and rounded to f32 (gpt-oss router). The per-token expert
// ids, and k = 4 at gpt-oss shape, come from PR #3579 "dasLLAMA gpt-oss arc" (fused MoE expert
// chain commit) and PR #3558 (section "gpt-oss: mx4 kernels to the lab-winning shape").
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kRoutePerLane = MOE_MAX_E / kWave;     // logits held per lane

// The top-k order is a total order of (value, id): a number before a NaN (a NaN logit ranks
// below every number, -inf included), the larger number first, equal values (-0.0 == +0.0) and
// two NaNs by the lower id. Being total, it gives every logit of a row a distinct rank, so the
// first k ranks always name k distinct experts in [0, E), whatever the row holds.
//
// It is computed through an integer key: a ranks before b exactly when key(a) > key(b). The high
// word maps the float monotonically onto unsigned integers (sign bit set: all bits inverted;
// clear: the sign bit set), -0 onto +0's word and every NaN onto 0, below -inf's 0x007FFFFF;
// the low word is ~id, so that the lower id is the larger key. Key 0 is below every key of a
// real (value, id) (whose low word is at least ~0x7FFFFFFF) and serves as "none". One 64-bit
// compare per pair keeps the rank loops on the vector ALU (boolean combinations of float
// compares become lane-mask logic on the scalar unit, a round trip per element).
__device__ __forceinline__ uint64_t rank_key(float v, int id) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t mag = b & 0x7FFFFFFFu;
  uint32_t hi = (b >> 31) ? ~b : (b | 0x80000000u);
  hi = mag == 0u ? 0x80000000u : hi;          // -0 as +0
  hi = mag > 0x7F800000u ? 0u : hi;           // NaN below every number
  return ((uint64_t)hi << 32) | (uint64_t)(~(uint32_t)id);
}

__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return rank_key(va, ia) > rank_key(vb, ib);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// Logits of one row for wave_topk_select: lane l holds experts j*64 + l (0 past E); N values per
// lane cover E <= 64 N.
template <int N = kRoutePerLane>
__device__ __forceinline__ void wave_topk_load(const float* __restrict__ row, int E,
                                               float (&v)[N]) {
  const int lane = (int)(threadIdx.x & 63);
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int e = j * kWave + lane;
    v[j] = (e < E) ? row[e] : 0.0f;
  }
}

// The k best experts of one logits row (E <= MOE_MAX_E, k <= min(E, MOE_MAX_K)) held as by
// wave_topk_load. Lane r < k ends with the r-th pick in (my_id, my_v); other lanes' outputs are
// unspecified. k rounds of a wavefront arg-max over the lanes' best remaining keys; no LDS.
template <int N = kRoutePerLane>
__device__ __forceinline__ void wave_topk_select(const float (&v)[N], int E, int k,
                                                 int& my_id, float& my_v) {
  const int lane = (int)(threadIdx.x & 63);
  uint64_t key[N];   // 0: absent or already chosen
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int e = j * kWave + lane;
    key[j] = e < E ? rank_key(v[j], e) : 0u;
  }
  my_id = 0;
  my_v = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) best = key[j] > best ? key[j] : best;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const uint64_t o = shfl_xor_u64(best, m);
      best = o > best ? o : best;
    }
    const int id = (int)~(uint32_t)best;   // k <= E: a real key won
    const int jw = id >> 6, lw = id & 63;
    float cand = 0.0f;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      if (j == jw) {
        cand = v[j];
        if (lane == lw) key[j] = 0u;
      }
    }
    const float vw = __shfl(cand, lw);
    if (lane == r) {
      my_id = id;
      my_v = vw;
    }
  }
}

// The rank of every lane's key among the keys of lanes 0..n-1 (n <= 64; the number of larger
// ones), n or more for lanes >= n. Keys of real entries are nonzero (rank_key's low word is the
// complemented id). Every lane writes its key into the wavefront's 64 keys of LDS scratch, then
// reads all of them eight at a time (broadcast reads; the LDS operations of a wavefront complete
// in order) and counts the larger ones.
__device__ __forceinline__ int wave_rank_keys(uint64_t mk, uint64_t* keys, int n) {
  const int lane = (int)(threadIdx.x & 63);
  keys[lane] = lane < n ? mk : 0u;
  int rank = 0;
  for (int j0 = 0; j0 < n; j0 += 8) {   // j0 + 8 <= 64; keys past n are 0 and never count
    const ulonglong2 a0 = *reinterpret_cast<const ulonglong2*>(keys + j0);
    const ulonglong2 a1 = *reinterpret_cast<const ulonglong2*>(keys + j0 + 2);
    const ulonglong2 a2 = *reinterpret_cast<const ulonglong2*>(keys + j0 + 4);
    const ulonglong2 a3 = *reinterpret_cast<const ulonglong2*>(keys + j0 + 6);
    rank += (a0.x > mk) + (a0.y > mk) + (a1.x > mk) + (a1.y > mk) + (a2.x > mk) +
            (a2.y > mk) + (a3.x > mk) + (a3.y > mk);
  }
  return lane < n ? rank : n + lane;
}

// E <= 64: the rank of every lane's logit among the row's E logits (the number that rank before
// it), the lane of rank r holding pick r; E or more for lanes >= E. From the logits row staged in
// LDS (row[0..63]; what lies past E is never compared) and 64 keys of LDS scratch of the calling
// wavefront.
__device__ __forceinline__ int wave_rank_lds(const float* row, uint64_t* keys, int E) {
  const int lane = (int)(threadIdx.x & 63);
  return wave_rank_keys(rank_key(row[lane], lane), keys, E);
}

// The same ranks from a logits row in memory (E <= 64): eight values per step by loads every
// lane makes at the same address, then the tail one at a time, so nothing past E is read.
__device__ __forceinline__ int wave_rank_row(const float* __restrict__ row, int E) {
  const int lane = (int)(threadIdx.x & 63);
  const uint64_t mk = rank_key(lane < E ? row[lane] : 0.0f, lane);
  int rank = 0;
  int j0 = 0;
  for (; j0 + 8 <= E; j0 += 8) {
    float vj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) vj[u] = row[j0 + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) rank += rank_key(vj[u], j0 + u) > mk;
  }
  for (; j0 < E; ++j0) rank += rank_key(row[j0], j0) > mk;
  return lane < E ? rank : E + lane;
}

// Expert of pick `slot` from wave_rank_lds / wave_rank_row ranks (uniform).
__device__ __forceinline__ int rank_pick(int rank, int slot) {
  return __ffsll((unsigned long long)__ballot(rank == slot)) - 1;
}

// The k best experts of one logits row in memory (E <= MOE_MAX_E, k <= min(E, MOE_MAX_K)), by
// the total order of rank_key: lane r < k ends with the r-th pick in (my_id, my_v). E <= 64:
// one rank pass (wave_rank_row); more: k arg-max rounds over as few values per lane as E needs.
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, int& my_id,
                                          float& my_v) {
  if (E <= kWave) {
    const int lane = (int)(threadIdx.x & 63);
    const float v = lane < E ? row[lane] : 0.0f;
    const int rank = wave_rank_row(row, E);
    my_id = 0;
    my_v = 0.0f;
    for (int r = 0; r < k; ++r) {
      const int id = rank_pick(rank, r);
      const float vr = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), id));
      if (lane == r) {
        my_id = id;
        my_v = vr;
      }
    }
    return;
  }
  // as few values per lane as E needs: the arg-max rounds scan every one of them
  if (E <= 2 * kWave) {
    float v[2];
    wave_topk_load(row, E, v);
    wave_topk_select(v, E, k, my_id, my_v);
  } else if (E <= 4 * kWave) {
    float v[4];
    wave_topk_load(row, E, v);
    wave_topk_select(v, E, k, my_id, my_v);
  } else {
    float v[kRoutePerLane];
    wave_topk_load(row, E, v);
    wave_topk_select(v, E, k, my_id, my_v);
  }
}

// Routing weight of the pick held by this lane (lanes 0..k-1 of wave_topk): the softmax over the
// k picks, summed in double in pick order relative to pick 0, rounded to f32. Every lane must
// call it (it shuffles); lanes >= k get a value of no meaning.
__device__ __forceinline__ float topk_weight(float my_v, int k) {
  const float v0 = __shfl(my_v, 0);
  double den = 0.0;
  for (int r = 0; r < k; ++r) den += exp((double)__shfl(my_v, r) - (double)v0);
  return (float)(exp((double)my_v - (double)v0) / den);
}

__device__ __forceinline__ void write_topk(int my_id, float my_v, int k, int32_t* __restrict__ ids,
                                           float* __restrict__ w) {
  const int lane = (int)(threadIdx.x & 63);
  const float wt = topk_weight(my_v, k);
  if (lane < k) {
    ids[lane] = my_id;
    w[lane] = wt;
  }
}

}  // namespace moe
