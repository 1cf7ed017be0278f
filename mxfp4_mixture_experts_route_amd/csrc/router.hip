// moe_router: the router projection and the routing front of the chain in one launch:
// logits = x W_r^T + b_r (bf16 MFMA, fp32 accumulation), top-k + softmax weights per token, and
// the bucket/CSR with padded prefix bases over all tokens.
//
// Sources: PR #3579 "dasLLAMA gpt-oss arc" (fused MoE expert chain commit: per-token expert ids
// in slot order; Metal fusion-lane commit: the bucket pass computes the padded-prefix bases
// itself instead of a separate prefix pass, the CSR unchanged bit for bit). The router itself is
// the gpt-oss linear layer with bias [ext]; the pages start from its output.
//
// gfx950 mapping. Workgroups of 16 wavefronts each take 16 tokens:
//  * logits: v_mfma_f32_16x16x32_bf16 with 16 router rows (experts) as the A operand and the 16
//    tokens as the B columns. A wavefront holds up to 4 expert tiles, which share each load of
//    the tokens' operand; the K = D reduction is split over the wavefronts that hold the same
//    tiles (16 / ceil(E/64) of them), whose partial tiles meet in LDS and are summed in a fixed
//    order, then the bias is added. Loads are buffer loads: tokens past T and experts past E
//    read zeros.
//  * top-k: one wavefront per token on the LDS logits row (the moe_route_topk code).
//  * bucket: the CSR needs every token's ids, so the LAST workgroup to finish its tokens builds
//    it: each workgroup stores its ids, and for each pick the number of earlier picks of the
//    same expert among its own 16 tokens (into pos[]), with device-scope stores, waits for them
//    to be acknowledged and increments a counter in the caller's workspace; the one that brings
//    it to the grid size resets the counter, reads every id and in-group count with
//    device-coherent loads (all in flight), histograms the picks per group in LDS, scans the
//    histograms over the groups and the padded counts over the experts, and places every pick
//    at base[e] + (picks of e in earlier groups) + (its in-group count). When the per-group table
//    does not fit its LDS budget, each wavefront instead sweeps all ids for whole experts in
//    ascending token order (one ballot per 64 tokens). No workgroup ever waits for another. The
//    tail is inlined into each kernel so that its LDS and global accesses keep their address
//    spaces (as a called function they become flat accesses, whose stores hold up every later
//    LDS wait).
//  * E >= 64 (and the pairs' grid within one round over the CUs): each 16-token group is routed
//    by a pair of workgroups with half of the experts each, so each streams half of W_r; each
//    takes the top k of its half, stores those candidates in the workspace and counts itself in
//    on its group's word; the later of the pair merges both halves' candidates under the same
//    order (the top k of the union of the halves' top k is the row's top k) and goes on as one.
//  * A few tokens (T <= 16, one token tile): the reduction is split over up to 48 workgroups of
//    4 wavefronts instead (one workgroup alone would read all the router rows from one CU, at a
//    small fraction of the chip's rate); their partial logits meet in the workspace, summed in
//    split order by the workgroup that completes the count, which then routes and builds the
//    CSR from its own LDS.
#include <algorithm>

#include "route_core.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kRtWaves = 16;
constexpr int kRtThreads = kRtWaves * kWave;
constexpr int kRtTok = 16;   // tokens per workgroup
constexpr int kSpWaves = 4;  // split kernel: wavefronts per workgroup
constexpr int kSpThreads = kSpWaves * kWave;
constexpr int kSpMaxSplit = 48;
// workspace words: [0] the completion counter; [kRtGrpOff, +kRtMaxGroups) the expert-split
// pairs' counters (zero between calls); from kRtDataOff, the split kernel's partial logits or
// the expert-split halves' candidates
constexpr int kRtGrpOff = 64;
constexpr int kRtMaxGroups = MOE_ROUTER_MAX_ROUTED / 16;
constexpr int kRtDataOff = kRtGrpOff + kRtMaxGroups;
constexpr int kRtParts = 2;   // expert split of the many-token kernel
static_assert(kRtDataOff + kRtParts * 2 * (MOE_ROUTER_MAX_ROUTED + 15 * MOE_MAX_K) <=
                  MOE_ROUTER_WS_WORDS, "router workspace");

constexpr int kRtTpw = 4;    // expert tiles per wavefront in the logits stage of router_kernel

// expert tiles, their groups of kRtTpw and the K split of the logits stage (a wavefront per
// tile group and K slice)
__host__ __device__ inline int rt_tiles(int E) { return (E + 15) / 16; }
// Parts of the expert split: with several workgroups (T > 16), E >= 64 (W_r large enough that
// streaming half of it pays for the merge) and the pairs' grid within one round over the CUs,
// each 16-token group is routed by a pair of workgroups holding half of the experts each (so
// each streams half of W_r), whose top-k candidates the later one of the pair merges.
__host__ inline int rt_parts(int64_t T, int E, int cus) {
  return (T > kRtTok && E >= 64 && (T + kRtTok - 1) / kRtTok * kRtParts <= cus) ? kRtParts : 1;
}
__host__ __device__ inline int rt_part_experts(int E, int P) { return (E + P - 1) / P; }
__host__ __device__ inline int rt_tgroups(int E) { return (rt_tiles(E) + kRtTpw - 1) / kRtTpw; }
__host__ __device__ inline int rt_ksplit(int E) {
  const int n = rt_tgroups(E);
  return n >= kRtWaves ? 1 : kRtWaves / n;
}
// The last workgroup's CSR over many tokens: per-group histograms of the picks (a group = one
// workgroup's 16 tokens), two experts per 32-bit word, when they fit this many bytes of LDS;
// otherwise every expert sweeps all ids.
constexpr int kGrpTableBytes = 64 * 1024;
constexpr int kGrpMaxSeg = 32;   // segments of the prefix over groups
__host__ __device__ inline int rt_groups(int64_t T) { return (int)((T + kRtTok - 1) / kRtTok); }
__host__ __device__ inline bool rt_grouped(int G, int E) {
  return G > 1 && (int64_t)G * ((E + 1) / 2) * 4 <= kGrpTableBytes;
}
// LDS of the CSR stage: the group table, expert counts and bases and the segment totals; or the
// counts, bases and every id
__host__ __device__ inline size_t rt_csr_bytes(int E, int64_t T, int k) {
  const int G = rt_groups(T);
  if (rt_grouped(G, E)) return ((size_t)G * ((E + 1) / 2) + 2 * E + kRtThreads) * sizeof(int);
  return (size_t)(2 * E + T * k) * sizeof(int);
}
// dynamic LDS: the logits stage's partial tiles or the CSR stage's arrays (row reads of the rank
// may run up to 63 floats past a row), then 512 B of rank keys per wavefront
__host__ __device__ inline size_t rt_keys_off(size_t rows_bytes, size_t csr_bytes) {
  const size_t p1 = rows_bytes + kWave * sizeof(float);
  return ((p1 > csr_bytes ? p1 : csr_bytes) + 15) & ~(size_t)15;
}
__host__ inline size_t rt_lds_bytes(int E, int64_t T, int k, int P) {
  const int En = rt_part_experts(E, P);   // the logits rows hold a part's experts
  return rt_keys_off((size_t)rt_ksplit(En) * kRtTok * En * sizeof(float), rt_csr_bytes(E, T, k)) +
         (size_t)kRtWaves * kWave * sizeof(uint64_t);
}
// an upper bound of rt_lds_bytes over every accepted shape
__host__ inline size_t rt_lds_most() {
  const size_t rows = (size_t)kRtTok * MOE_MAX_E * sizeof(float);   // ksplit*E <= 1024
  const size_t grouped = kGrpTableBytes + (2 * MOE_MAX_E + kRtThreads) * sizeof(int);
  const size_t sweep = (2 * MOE_MAX_E + MOE_ROUTER_MAX_ROUTED) * sizeof(int);
  return rt_keys_off(rows, grouped > sweep ? grouped : sweep) +
         (size_t)kRtWaves * kWave * sizeof(uint64_t);
}
// split kernel: the tile's logits rows, or the CSR stage's arrays; then the keys
__host__ inline size_t sp_lds_bytes(int E, int64_t T, int k) {
  return rt_keys_off((size_t)kRtTok * E * sizeof(float), (size_t)(2 * E + T * k) * sizeof(int)) +
         (size_t)kSpWaves * kWave * sizeof(uint64_t);
}

// 16 x 16 logits tile of (16 experts from e_row0, 16 tokens from t0) over k steps [s0, s1) of
// 32: MFMA with the router rows as A and the tokens as B; lane (lr, lg) ends with experts
// e_row0 + 4lg..+3 of token t0 + lr. 8 steps per round, all 16 loads in flight before the
// MFMAs; steps past s1, experts past E and tokens past T read zeros.
__device__ __forceinline__ f32x4_t router_tile(__amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx,
                                               int D, int E, int T, int e_row0, int t0, int s0,
                                               int s1) {
  const int lane = (int)(threadIdx.x & 63), lr = lane & 15, lg = lane >> 4;
  const int e_row = e_row0 + lr;
  const uint32_t ao = e_row < E ? ((uint32_t)e_row * D + 8 * lg) * 2 : kOOB;
  const uint32_t bo = t0 + lr < T ? ((uint32_t)(t0 + lr) * D + 8 * lg) * 2 : kOOB;
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int sb = s0; sb < s1; sb += 8) {
    u32x4_t a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = sb + i < s1;
      a[i] = buf_load16(rw, ok ? ao : kOOB, (uint32_t)(sb + i) * 64);
      b[i] = buf_load16(rx, ok ? bo : kOOB, (uint32_t)(sb + i) * 64);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bf16x8_t A, B;
      __builtin_memcpy(&A, &a[i], 16);
      __builtin_memcpy(&B, &b[i], 16);
      if (i & 1)
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc1, 0, 0, 0);
      else
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc0, 0, 0, 0);
    }
  }
  return acc0 + acc1;
}

// Exclusive scan of the padded counts cnt[0..E) into base[] and basep[], counts[] = cnt (E <=
// the workgroup's threads); returns the padded total. Ends with a barrier.
__device__ __forceinline__ int csr_bases(const int* cnt, int* base, int E, int tile_m,
                                         int32_t* __restrict__ counts, int32_t* __restrict__ basep,
                                         int* wave_tot) {
  const int tid = (int)threadIdx.x, nthreads = (int)blockDim.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), waves = nthreads >> 6;
  const int c = tid < E ? cnt[tid] : 0;
  const int padded = (c + tile_m - 1) / tile_m * tile_m;
  int incl = padded;
  for (int m = 1; m < 64; m <<= 1) {
    const int o = __shfl_up(incl, m);
    if (lane >= m) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int v = 0; v < waves; ++v) {
    if (v < wave) before += wave_tot[v];
    total += wave_tot[v];
  }
  const int excl = before + incl - padded;
  if (tid < E) {
    base[tid] = excl;
    counts[tid] = c;
    basep[tid] = excl;
  }
  if (tid == 0) basep[E] = total;
  __syncthreads();
  return total;
}

// Padding rows of every expert (wavefront per expert), then the ghost rows up to mpad_max.
__device__ __forceinline__ void csr_pad(const int* cnt, const int* base, int E, int tile_m,
                                        int total, int mpad_max, int32_t* __restrict__ row_tok) {
  const int tid = (int)threadIdx.x, nthreads = (int)blockDim.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), waves = nthreads >> 6;
  for (int e = wave; e < E; e += waves) {
    const int c = cnt[e], b = base[e];
    const int pe = (c + tile_m - 1) / tile_m * tile_m;
    for (int j = c + lane; j < pe; j += 64) row_tok[b + j] = -1;
  }
  for (int r = total + tid; r < mpad_max; r += nthreads) row_tok[r] = -1;
}

// The routing of tokens t0.. (at most 16) from their logits rows in LDS (part[tok][En], experts
// e_lo..e_lo+En-1 of E), then the CSR by the workgroup that holds the last picks. counter: the
// caller's completion word when several workgroups route (the one that completes the count
// builds the CSR from the ids in memory), or NULL when this workgroup routes every token (the
// ids are in its LDS). With an expert split (P = 2 parts, part `part` of group g), each
// workgroup first takes the top k of its own experts, stores those candidates in the workspace
// (cand) and counts itself in on its group's word (grp); the one that completes the pair merges
// both parts' candidates under the same order (the top k of the union of each part's top k is
// the top k of the row) and goes on alone; the other leaves.
// keys: 512 B of LDS per wavefront for the ranks (E <= 64 rows, the merge).
//
// The CSR row of pick (t, s) routed to expert e is base[e] plus the number of earlier tokens
// routed to e (a token picks an expert at most once). With several workgroups (groups of 16
// tokens) that number splits into the picks of e in earlier groups plus those of earlier tokens
// of the same group: each workgroup counts the latter for its own picks and leaves them in pos[]
// (device-scope stores, like the ids); the last workgroup histograms the picks per group in
// LDS, scans the histograms over the groups, and places every pick at once. When the group
// table does not fit, each wavefront of the last workgroup sweeps all ids for its experts.
__device__ __forceinline__ void router_tail(float* part, int T, int t0, int E, int En, int e_lo,
                                            int k, int tile_m, int mpad_max,
                                            int32_t* __restrict__ ids, float* __restrict__ w,
                                            int32_t* __restrict__ counts,
                                            int32_t* __restrict__ basep,
                                            int32_t* __restrict__ row_tok,
                                            int32_t* __restrict__ pos, uint32_t* counter,
                                            int n_groups, int P, int pidx, int g, uint32_t* grp,
                                            uint32_t* cand, uint8_t* smem, uint64_t* keys) {
  __shared__ int s_last;
  __shared__ __attribute__((aligned(16))) int s_ids[kRtTok * MOE_MAX_K];   // this group's picks
  __shared__ float s_pv[kRtTok * MOE_MAX_K];                                // their logits
  __shared__ int s_wave_tot[kRtWaves];
  const int tid = (int)threadIdx.x, nthreads = (int)blockDim.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), waves = nthreads >> 6;
  const int ntok = min(kRtTok, T - t0);

  // ---- top-k of this workgroup's experts: wavefront w takes tokens t0 + w, t0 + w + waves, ...
  for (int tt = wave; tt < ntok; tt += waves) {
    int my_id = 0;
    float my_v;
    const float* row = part + (size_t)tt * En;
    if (En <= kWave) {   // rank against the row's keys in LDS (row[lane] read for every lane)
      const int rank = wave_rank_lds(row, keys + (size_t)wave * kWave, En);
      for (int r = 0; r < k; ++r) {
        const int id = rank_pick(rank, r);
        if (lane == r) my_id = id;
      }
      my_v = row[min(max(my_id, 0), kWave - 1)];
    } else {
      wave_topk(row, En, k, my_id, my_v);
    }
    if (lane < k) {
      s_ids[tt * k + lane] = e_lo + my_id;
      s_pv[tt * k + lane] = my_v;
    }
  }
  __syncthreads();

  if (P > 1) {
    // this part's candidates into the workspace (device-scope stores), acknowledged, then the
    // pair's count; the workgroup that completes it merges
    uint32_t* const mine = cand + (size_t)(g * P + pidx) * kRtTok * k * 2;
    for (int i = tid; i < ntok * k; i += nthreads) {
      __hip_atomic_store(mine + 2 * i, __float_as_uint(s_pv[i]), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(mine + 2 * i + 1, (uint32_t)s_ids[i], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(grp + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               (uint32_t)P - 1;
    __syncthreads();
    if (!s_last) return;
    if (tid == 0)   // ready for the next call
      __hip_atomic_store(grp + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // merge: per token, lane j < P*k holds candidate j (part j / k, pick j % k), read with
    // device-coherent loads; its rank among them by the same key gives the final picks
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(cand + (size_t)g * P * kRtTok * k * 2, (uint32_t)(P * kRtTok * k * 8));
    const int n = P * k;
    for (int tt = wave; tt < ntok; tt += waves) {
      float cv = 0.0f;
      int cid = 0;
      uint64_t mk = 0;
      if (lane < n) {
        const int pp = lane / k, r = lane - pp * k;
        const uint32_t off = (uint32_t)(((pp * kRtTok + tt) * k + r) * 8);
        cv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc, off, 0, 16));
        cid = (int)__builtin_amdgcn_raw_buffer_load_b32(rc, off + 4, 0, 16);
        mk = rank_key(cv, cid);
      }
      const int rank = wave_rank_keys(mk, keys + (size_t)wave * kWave, n);
      for (int r = 0; r < k; ++r) {
        const int src = rank_pick(rank, r);
        const int id = __shfl(cid, src);
        const float v = __shfl(cv, src);
        if (lane == r) {
          s_ids[tt * k + r] = id;
          s_pv[tt * k + r] = v;
        }
      }
    }
    __syncthreads();
  }

  // ---- the picks: weights (softmax over the k picks), ids with device-scope atomic stores
  // (they bypass the XCD's non-coherent L2, so that another XCD's workgroup can read them)
  for (int tt = wave; tt < ntok; tt += waves) {
    const int my_id = lane < k ? s_ids[tt * k + lane] : 0;
    const float my_v = lane < k ? s_pv[tt * k + lane] : 0.0f;
    const float wt = topk_weight(my_v, k);
    if (lane < k) {
      __hip_atomic_store(ids + (size_t)(t0 + tt) * k + lane, my_id, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      w[(size_t)(t0 + tt) * k + lane] = wt;
    }
  }
  const int R = T * k;
  const bool alone = counter == nullptr;
  __syncthreads();

  if (alone) {
    // every routed row at once, its rank counted over the earlier picks in LDS; then the padding
    int* cnt = reinterpret_cast<int*>(smem);
    int* base = cnt + E;
    for (int i = tid; i < E; i += nthreads) cnt[i] = 0;
    __syncthreads();
    for (int i = tid; i < R; i += nthreads)
      if ((unsigned)s_ids[i] < (unsigned)E) atomicAdd(&cnt[s_ids[i]], 1);
    __syncthreads();
    const int total = csr_bases(cnt, base, E, tile_m, counts, basep, s_wave_tot);
    for (int r = tid; r < R; r += nthreads) {
      const int e = s_ids[r], t = r / k;
      if ((unsigned)e >= (unsigned)E) continue;
      int rank = 0;
      for (int r2 = 0; r2 < t * k; ++r2) rank += s_ids[r2] == e;
      pos[r] = base[e] + rank;
      row_tok[base[e] + rank] = t0 + t;
    }
    csr_pad(cnt, base, E, tile_m, total, mpad_max, row_tok);
    return;
  }

  // ---- several workgroups: this group's in-group ranks, then the last one builds the CSR ----
  const int G = n_groups;
  const bool grouped = rt_grouped(G, E);
  if (grouped) {
    for (int i = tid; i < ntok * k; i += nthreads) {
      const int e = s_ids[i], before = (i / k) * k;
      int lr = 0, j = 0;
      for (; j + 4 <= before; j += 4) {
        const int4 v = *reinterpret_cast<const int4*>(s_ids + j);
        lr += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
      }
      for (; j < before; ++j) lr += s_ids[j] == e;
      __hip_atomic_store(pos + (size_t)t0 * k + i, lr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Every wavefront waits until its stores are acknowledged, then the workgroup counts itself
  // in; the one that completes the count reads the ids (and in-group ranks) with device-coherent
  // loads (sc1, as the device-scope stores that wrote them), all in flight at once. (A
  // device-scope fence would also work but writes back and invalidates the whole L2, which
  // costs microseconds per workgroup.)
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)G - 1;
  __syncthreads();
  if (!s_last) return;
  if (tid == 0)   // ready for the next call
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  constexpr int kPer = MOE_ROUTER_MAX_ROUTED / kRtThreads;   // picks per thread: r = tid + i*1024
  const __amdgpu_buffer_rsrc_t rid = make_rsrc(ids, (uint32_t)R * 4);
  const __amdgpu_buffer_rsrc_t rpos = make_rsrc(pos, (uint32_t)R * 4);
  int my_e[kPer], my_lr[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    my_e[i] = -1;
    my_lr[i] = 0;
    if (i * kRtThreads < R) {   // uniform over the workgroup
      const int r = tid + i * kRtThreads;
      const uint32_t off = r < R ? (uint32_t)r * 4 : kOOB;
      my_e[i] = r < R ? (int)__builtin_amdgcn_raw_buffer_load_b32(rid, off, 0, 16) : -1;
      if (grouped) my_lr[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(rpos, off, 0, 16);
    }
  }

  if (grouped) {
    // LDS: tbl[G][EW] (experts 2w and 2w+1 in the low and high halves of word w), cnt[E],
    // base[E], seg[S][EW]
    const int EW = (E + 1) >> 1;
    uint32_t* tbl = reinterpret_cast<uint32_t*>(smem);
    int* cnt = reinterpret_cast<int*>(tbl + (size_t)G * EW);
    int* base = cnt + E;
    uint32_t* seg = reinterpret_cast<uint32_t*>(base + E);
    for (int i = tid; i < G * EW; i += nthreads) tbl[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = my_e[i];
      if ((unsigned)e < (unsigned)E) {
        const int g = ((tid + i * kRtThreads) / k) / kRtTok;
        atomicAdd(&tbl[g * EW + (e >> 1)], (e & 1) ? 0x10000u : 1u);
      }
    }
    __syncthreads();
    // exclusive prefix of each column over the groups: S segments of L groups each (a half-word
    // never exceeds T <= MOE_ROUTER_MAX_ROUTED, so the halves do not carry into each other)
    const int S = min(min(nthreads / EW, kGrpMaxSeg), G);
    const int L = (G + S - 1) / S;
    const int col = tid % EW, sg = tid / EW;
    const int g0 = sg * L, g1 = min(G, g0 + L);
    if (sg < S) {
      uint32_t sum = 0;
      for (int g = g0; g < g1; ++g) sum += tbl[g * EW + col];
      seg[sg * EW + col] = sum;
    }
    __syncthreads();
    if (tid < EW) {
      uint32_t run = 0;
      for (int q = 0; q < S; ++q) {
        const uint32_t v = seg[q * EW + tid];
        seg[q * EW + tid] = run;
        run += v;
      }
      cnt[2 * tid] = (int)(run & 0xFFFFu);
      if (2 * tid + 1 < E) cnt[2 * tid + 1] = (int)(run >> 16);
    }
    __syncthreads();
    if (sg < S) {
      uint32_t run = seg[sg * EW + col];
      for (int g = g0; g < g1; ++g) {
        const uint32_t v = tbl[g * EW + col];
        tbl[g * EW + col] = run;
        run += v;
      }
    }
    __syncthreads();
    const int total = csr_bases(cnt, base, E, tile_m, counts, basep, s_wave_tot);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = my_e[i];
      if ((unsigned)e < (unsigned)E) {
        const int r = tid + i * kRtThreads, t = r / k;
        const uint32_t word = tbl[(t / kRtTok) * EW + (e >> 1)];
        const int row = base[e] + (int)((word >> ((e & 1) * 16)) & 0xFFFFu) + my_lr[i];
        pos[r] = row;
        row_tok[row] = t;
      }
    }
    csr_pad(cnt, base, E, tile_m, total, mpad_max, row_tok);
    return;
  }

  // the group table does not fit: every id into LDS, then wavefront v owns experts v, v +
  // waves, ... and sweeps all tokens in ascending order, one ballot per 64 tokens
  int* cnt = reinterpret_cast<int*>(smem);
  int* base = cnt + E;
  int* idl = base + E;
  for (int i = tid; i < E; i += nthreads) cnt[i] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = tid + i * kRtThreads, e = my_e[i];
    if (r < R) {
      idl[r] = e;
      if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  const int total = csr_bases(cnt, base, E, tile_m, counts, basep, s_wave_tot);
  for (int e = wave; e < E; e += waves) {
    const int b = base[e];
    int running = 0;
    for (int tt = 0; tt < T; tt += 64) {
      const int t = tt + lane;
      int slot = -1;
      if (t < T)
        for (int s = 0; s < k; ++s)
          if (idl[t * k + s] == e) slot = s;
      const uint64_t ballot = __ballot(slot >= 0);
      if (slot >= 0) {
        const int r = b + running + __popcll(ballot & (lane ? (~0ull >> (64 - lane)) : 0ull));
        row_tok[r] = t;
        pos[(size_t)t * k + slot] = r;
      }
      running += __popcll(ballot);
    }
  }
  csr_pad(cnt, base, E, tile_m, total, mpad_max, row_tok);
}

// nt <= kRtTpw logits tiles of 16 experts each (from e_row0, 16 apart) and the 16 tokens from
// t0, over k steps [s0, s1) of 32, as router_tile; the tokens' operand is loaded once per step
// and shared by the tiles (the wavefront's share of the workgroup's reads of x falls with the
// number of tiles it holds). 4 steps per round, all loads of a round in flight before its
// MFMAs, which alternate between the tiles' accumulators.
__device__ __forceinline__ void router_tiles(__amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx,
                                             int D, int E, int T, int e_row0, int nt, int t0,
                                             int s0, int s1, f32x4_t (&acc)[kRtTpw]) {
  const int lane = (int)(threadIdx.x & 63), lr = lane & 15, lg = lane >> 4;
  uint32_t ao[kRtTpw];
#pragma unroll
  for (int j = 0; j < kRtTpw; ++j) {
    const int e_row = e_row0 + 16 * j + lr;
    ao[j] = j < nt && e_row < E ? ((uint32_t)e_row * D + 8 * lg) * 2 : kOOB;
    acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t bo = t0 + lr < T ? ((uint32_t)(t0 + lr) * D + 8 * lg) * 2 : kOOB;
  for (int sb = s0; sb < s1; sb += 4) {
    u32x4_t a[kRtTpw][4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = sb + i < s1;
      b[i] = buf_load16(rx, ok ? bo : kOOB, (uint32_t)(sb + i) * 64);
#pragma unroll
      for (int j = 0; j < kRtTpw; ++j)
        if (j < nt) a[j][i] = buf_load16(rw, ok ? ao[j] : kOOB, (uint32_t)(sb + i) * 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x8_t B;
      __builtin_memcpy(&B, &b[i], 16);
#pragma unroll
      for (int j = 0; j < kRtTpw; ++j)
        if (j < nt) {
          bf16x8_t A;
          __builtin_memcpy(&A, &a[j][i], 16);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[j], 0, 0, 0);
        }
    }
  }
}

// Workgroups of 16 wavefronts each take 16 tokens over the whole reduction, and the experts of
// one part (P parts; workgroup L: group L / P, part L % P).
__global__ void __launch_bounds__(kRtThreads)
router_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
              const float* __restrict__ br, int T, int D, int E, int k, int tile_m,
              int mpad_max, float* __restrict__ logits, int32_t* __restrict__ ids,
              float* __restrict__ w, int32_t* __restrict__ counts, int32_t* __restrict__ basep,
              int32_t* __restrict__ row_tok, int32_t* __restrict__ pos,
              uint32_t* __restrict__ ws, int P) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int g = (int)blockIdx.x / P, pidx = (int)blockIdx.x - g * P;
  const int G = (int)gridDim.x / P;
  const int t0 = g * kRtTok;
  const int Ep = rt_part_experts(E, P), e_lo = pidx * Ep, En = min(Ep, E - e_lo);
  const int ntiles = rt_tiles(En), ntg = rt_tgroups(En), ksplit = rt_ksplit(En);
  const int KS = D >> 5;   // 32-wide k steps
  float* part = reinterpret_cast<float*>(smem);   // [ksplit][kRtTok][En]

  // ---- logits of the workgroup's 16 tokens and En experts: a wavefront per (tile group, K
  // slice) ----
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wr + (size_t)e_lo * D, (uint32_t)En * D * 2);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)T * D * 2);
  for (int u = wave; u < ntg * ksplit; u += kRtWaves) {
    const int tg = u % ntg, p = u / ntg;
    const int nt = min(kRtTpw, ntiles - tg * kRtTpw);
    f32x4_t acc[kRtTpw];
    router_tiles(rw, rx, D, En, T, tg * kRtTpw * 16, nt, t0, p * KS / ksplit,
                 (p + 1) * KS / ksplit, acc);
#pragma unroll
    for (int j = 0; j < kRtTpw; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = (tg * kRtTpw + j) * 16 + 4 * lg + i;
        if (j < nt && e < En) part[((size_t)p * kRtTok + lr) * En + e] = acc[j][i];
      }
  }
  __syncthreads();
  for (int i = tid; i < kRtTok * En; i += kRtThreads) {
    const int tok = i / En, e = i - tok * En;
    float v = part[(size_t)tok * En + e];
    for (int p = 1; p < ksplit; ++p) v += part[((size_t)p * kRtTok + tok) * En + e];
    if (br) v += br[e_lo + e];
    part[(size_t)tok * En + e] = v;   // only this thread touches element (tok, e)
    if (logits && t0 + tok < T) logits[(size_t)(t0 + tok) * E + e_lo + e] = v;
  }
  __syncthreads();
  uint64_t* const keys = reinterpret_cast<uint64_t*>(
      smem + rt_keys_off((size_t)ksplit * kRtTok * En * sizeof(float), rt_csr_bytes(E, T, k)));
  router_tail(part, T, t0, E, En, e_lo, k, tile_m, mpad_max, ids, w, counts, basep, row_tok, pos,
              gridDim.x == 1 ? nullptr : ws, G, P, pidx, g, ws + kRtGrpOff, ws + kRtDataOff, smem,
              keys);
}

// A few tokens (T <= 16, E <= 256): the reduction split over `nsplit` small workgroups, so that
// the router rows stream from many CUs at once (one CU alone reads them at a fraction of the
// chip's rate). Workgroup s takes k steps [s*KS/nsplit, (s+1)*KS/nsplit) of every expert tile
// and stores its partial logits [T][E] in the workspace (device-scope stores); the workgroup
// that completes the count sums the partials in split order, adds the bias and routes every
// token, then builds the CSR from its own LDS.
__global__ void __launch_bounds__(kSpThreads)
router_split_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                    const float* __restrict__ br, int T, int D, int E, int k, int tile_m,
                    int mpad_max, float* __restrict__ logits, int32_t* __restrict__ ids,
                    float* __restrict__ w, int32_t* __restrict__ counts,
                    int32_t* __restrict__ basep, int32_t* __restrict__ row_tok,
                    int32_t* __restrict__ pos, uint32_t* __restrict__ ws, int nsplit) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_last;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int s = (int)blockIdx.x;
  const int KS = D >> 5;
  float* const partg = reinterpret_cast<float*>(ws + kRtDataOff);   // [nsplit][T][E]
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wr, (uint32_t)E * D * 2);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)T * D * 2);
  for (int tile = wave; tile < rt_tiles(E); tile += kSpWaves) {
    const f32x4_t acc = router_tile(rw, rx, D, E, T, tile * 16, 0, s * KS / nsplit,
                                    (s + 1) * KS / nsplit);
    if (lr < T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tile * 16 + 4 * lg + i;
        if (e < E)
          __hip_atomic_store(partg + ((size_t)s * T + lr) * E + e, acc[i], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // the partials are acknowledged
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(ws, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)nsplit - 1;
  __syncthreads();
  if (!s_last) return;
  // the last workgroup: logits = sum of the partials in split order, then the bias. The
  // partials are read with the device-coherent bit (sc1, as the device-scope stores that wrote
  // them), as plain loads: all in flight at once (atomic loads would be issued one at a time)
  float* part = reinterpret_cast<float*>(smem);   // [kRtTok][E]
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(partg, (uint32_t)nsplit * T * E * 4);
  for (int i = tid; i < T * E; i += kSpThreads) {
    const int tok = i / E, e = i - tok * E;
    float pv[kSpMaxSplit];
#pragma unroll
    for (int s2 = 0; s2 < kSpMaxSplit; ++s2)
      pv[s2] = s2 < nsplit ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                 rp, (uint32_t)(((s2 * T + tok) * E + e) * 4), 0, 16))
                           : 0.0f;
    float v = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < kSpMaxSplit; ++s2)
      if (s2 < nsplit) v += pv[s2];
    if (br) v += br[e];
    part[(size_t)tok * E + e] = v;
    if (logits) logits[(size_t)tok * E + e] = v;
  }
  if (tid == 0) __hip_atomic_store(ws, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  uint64_t* const keys = reinterpret_cast<uint64_t*>(
      smem + rt_keys_off((size_t)kRtTok * E * sizeof(float), (size_t)(2 * E + T * k) * sizeof(int)));
  router_tail(part, T, 0, E, E, 0, k, tile_m, mpad_max, ids, w, counts, basep, row_tok, pos,
              nullptr, 1, 1, 0, 0, nullptr, nullptr, smem, keys);
}

}  // namespace moe

extern "C" int moe_router(const uint16_t* x, const uint16_t* w_r, const float* b_r, int64_t T,
                          int D, int E, int k, int tile_m, int64_t mpad_max, float* logits,
                          int32_t* ids, float* w, int32_t* counts, int32_t* basep,
                          int32_t* row_tok, int32_t* pos, uint32_t* ws, void* stream) {
  if (!x || !w_r || !ids || !w || !counts || !basep || !row_tok || !pos || !ws || T < 1 ||
      D < 1 || E < 1 || k < 1 || k > E || k > MOE_MAX_K)
    return MOE_EINVAL;
  if (E > MOE_MAX_E || D % 32 != 0 || T * k > MOE_ROUTER_MAX_ROUTED || tile_m < 1 ||
      tile_m > MOE_MAX_TILE_M || T * (int64_t)D * 2 >= (1LL << 31) ||
      (int64_t)E * D * 2 >= (1LL << 31))
    return MOE_ESHAPE;
  const int64_t need = moe_mpad_max(T, k, E, tile_m);
  if (mpad_max < need || mpad_max > 0x7FFFFFFFLL) return MOE_ESHAPE;
  if ((((uintptr_t)x) & 15) || (((uintptr_t)w_r) & 15) || (((uintptr_t)ws) & 3))
    return MOE_EALIGN;
  // a few tokens: the reduction split over workgroups whose partials fit the workspace
  const int KS = D / 32;
  int nsplit = 0;
  if (T <= moe::kRtTok && E <= moe::kSpThreads) {
    const int64_t cap = (MOE_ROUTER_WS_WORDS - moe::kRtDataOff) / (T * (int64_t)E);
    nsplit = (int)std::min<int64_t>(std::min<int64_t>(cap, KS), moe::kSpMaxSplit);
  }
  if (nsplit >= 2) {
    moe::launch(moe::router_split_kernel, dim3((unsigned)nsplit), dim3(moe::kSpThreads),
                (unsigned)moe::sp_lds_bytes(E, T, k), (hipStream_t)stream, x, w_r, b_r, (int)T, D,
                E, k, tile_m, (int)mpad_max, logits, ids, w, counts, basep, row_tok, pos, ws,
                nsplit);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
  }
  static int cus_of[moe::kMaxDevices] = {};
  const int dslot = moe::device_slot();
  int cus = dslot >= 0 ? cus_of[dslot] : 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return MOE_ELAUNCH;
    if (dslot >= 0) cus_of[dslot] = cus;
  }
  const int P = moe::rt_parts(T, E, cus);
  const size_t lds = moe::rt_lds_bytes(E, T, k, P);
  static bool lds_attr_set[moe::kMaxDevices] = {};   // > 64 KB of LDS: opt in once per device
  if (dslot < 0 || !lds_attr_set[dslot]) {
    const size_t most = moe::rt_lds_most();
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&moe::router_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)most) != hipSuccess)
      return MOE_ELAUNCH;
    if (dslot >= 0) lds_attr_set[dslot] = true;
  }
  const int64_t blocks = (T + moe::kRtTok - 1) / moe::kRtTok * P;
  moe::launch(moe::router_kernel, dim3((unsigned)blocks), dim3(moe::kRtThreads), (unsigned)lds,
              (hipStream_t)stream, x, w_r, b_r, (int)T, D, E, k, tile_m, (int)mpad_max, logits,
              ids, w, counts, basep, row_tok, pos, ws, P);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
