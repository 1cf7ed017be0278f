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

// a ranks before b in a total order of (value, id): a number before a NaN (a NaN logit ranks
// below every number, -inf included), the larger number first, equal values (-0.0 == +0.0) and
// two NaNs by the lower id. Being total, it gives every logit of a row a distinct rank, so the
// first k ranks always name k distinct experts in [0, E), whatever the row holds.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  const bool na = va != va, nb = vb != vb;
  const bool lower_id = ia < ib;
  return (nb & (!na | lower_id)) | (!na & !nb & ((va > vb) | ((va == vb) & lower_id)));
}

// Logits of one row for wave_topk_select: lane l holds experts j*64 + l (0 past E).
__device__ __forceinline__ void wave_topk_load(const float* __restrict__ row, int E,
                                               float (&v)[kRoutePerLane]) {
  const int lane = (int)(threadIdx.x & 63);
#pragma unroll
  for (int j = 0; j < kRoutePerLane; ++j) {
    const int e = j * kWave + lane;
    v[j] = (e < E) ? row[e] : 0.0f;
  }
}

// The k best experts of one logits row (E <= MOE_MAX_E, k <= min(E, MOE_MAX_K)) held as by
// wave_topk_load. Lane r < k ends with the r-th pick in (my_id, my_v); other lanes' outputs are
// unspecified. k rounds of a wavefront arg-best over per-lane candidates; no LDS.
__device__ __forceinline__ void wave_topk_select(const float (&v)[kRoutePerLane], int E, int k,
                                                 int& my_id, float& my_v) {
  const int lane = (int)(threadIdx.x & 63);
  uint32_t taken = 0;                 // bit j: expert j*64+lane already chosen (or absent)
#pragma unroll
  for (int j = 0; j < kRoutePerLane; ++j)
    if (j * kWave + lane >= E) taken |= 1u << j;

  my_id = 0;
  my_v = 0.0f;
  for (int r = 0; r < k; ++r) {
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
    if (lane == r) {
      my_id = bi;
      my_v = bv;
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
  }
}

// E <= 64: the rank of every lane's logit among the row's E logits (the number that rank before
// it), the lane of rank r holding pick r; E or more for lanes >= E. From the logits row staged in
// LDS (row[0..63]; what lies past E is never compared): eight values per step come as broadcast
// LDS reads and every compare is independent of the previous one, so the steps overlap. (A
// broadcast of each lane's value by v_readlane waits for the scalar register every step:
// ~115 cycles a step, 1.5 us for E = 32.)
__device__ __forceinline__ int wave_rank_lds(const float* row, int E) {
  const int lane = (int)(threadIdx.x & 63);
  const float v = row[lane];
  int rank = 0;
  for (int j0 = 0; j0 < E; j0 += 8) {
    const float4 a = *reinterpret_cast<const float4*>(row + j0);
    const float4 b = *reinterpret_cast<const float4*>(row + j0 + 4);
    const float vj[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int u = 0; u < 8; ++u)
      rank += (j0 + u < E && ranks_before(vj[u], j0 + u, v, lane)) ? 1 : 0;
  }
  return lane < E ? rank : E + lane;
}

// The same ranks from a logits row in memory (global or LDS; E <= 64): eight values per step
// by loads every lane makes at the same address, then the tail one at a time, so nothing past
// E is read and the compares are independent of each other (no cross-lane step in the chain).
__device__ __forceinline__ int wave_rank_row(const float* __restrict__ row, int E) {
  const int lane = (int)(threadIdx.x & 63);
  const float v = lane < E ? row[lane] : 0.0f;
  int rank = 0;
  int j0 = 0;
  for (; j0 + 8 <= E; j0 += 8) {
    float vj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) vj[u] = row[j0 + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) rank += ranks_before(vj[u], j0 + u, v, lane) ? 1 : 0;
  }
  for (; j0 < E; ++j0) rank += ranks_before(row[j0], j0, v, lane) ? 1 : 0;
  return lane < E ? rank : E + lane;
}

// Expert of pick `slot` from wave_rank_lds / wave_rank_row ranks (uniform).
__device__ __forceinline__ int rank_pick(int rank, int slot) {
  return __ffsll((unsigned long long)__ballot(rank == slot)) - 1;
}

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
  float v[kRoutePerLane];
  wave_topk_load(row, E, v);
  wave_topk_select(v, E, k, my_id, my_v);
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
