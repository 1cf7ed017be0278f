/*
 * moe_mx4.h — C ABI of the routed MXFP4 mixture-of-experts chain for MI355X (gfx950).
 *
 * The chain (gpt-oss routed experts) runs as five stream-ordered calls:
 *
 *   moe_route_topk  logits -> top-k expert ids + routing weights
 *   moe_router      x -> router logits, ids, weights and the CSR in one launch (the router
 *                   projection fused with moe_route_topk and moe_bucket)
 *   moe_bucket      ids    -> CSR of routed rows per expert with padded prefix bases
 *   mx4_pack_experts  one-time repack of MXFP4 expert weights into the GPU's chunked layout
 *   mx4_moe_gemv    gate_up / down MXFP4 projection, few rows per expert (decode)
 *   mx4_moe_gemm    the same function on MFMA, many rows per expert (prefill)
 *   moe_combine     router-weighted sum of each token's expert rows, in slot order
 *
 * with MXFP8 activations on the MX-scaled MFMA (a variant; formats from the OCP specs):
 *
 *   mx8_quantize      bf16 rows -> MXFP8 rows (E4M3 + one e8m0 scale per 32 values)
 *   mx4_moe_gemm_mx8  the projection of mx4_moe_gemm over MXFP8 activation rows
 *
 * and, for decode (a few tokens), the same chain fused into two launches:
 *
 *   mx4_moe_decode  logits + x -> routing, CSR, h, (d), y
 *   mx4_moe_decode_persistent  the same in one launch (a resident grid; down weights stream
 *                   while gate_up is still running)
 *   mx4_moe_decode_persistent_static  the same with a library-held workspace (no allocation)
 *
 * Sources (web pages on the daScript repository's dasLLAMA engine; cited by tag below):
 *   [fusion]  PR #3579 "dasLLAMA gpt-oss arc", commit log, the Metal fusion-lane commit: the
 *             bucket pass computes each expert's padded-prefix base inside its workgroup and
 *             publishes it (the separate prefix pass is gone, the CSR is unchanged bit for bit);
 *             the expert matmul starts its accumulators from the expert's bias row; the prefill
 *             SwiGLU-OAI skips ghost rows beyond the last bucket's padded end.
 *   [chain]   PR #3579, commit log, the fused MoE expert chain commit, and the PR body's section
 *             "Fused MoE expert chain": stage 0 = gate and up rows + bias + activation, stage 1 =
 *             down rows + bias, then the routing-weighted sum taken in slot order.
 *   [mx4]     PR #3558 "dasLLAMA: dig the last two board reds green", section "gpt-oss: mx4
 *             kernels to the lab-winning shape" and its ladder table: MXFP4 weights decoded via
 *             a 16-entry e2m1 table and one e8m0 exponent byte per 32-value block, bit-exact for
 *             every one of the 256 exponent bytes; gpt-oss shapes E=32, nfe=dim=2880, k=4.
 *
 * Conventions shared by every call
 *   - All pointers other than the `mx4_experts` descriptor itself are DEVICE pointers owned by
 *     the caller. The library never allocates or frees device memory and keeps no per-call state.
 *   - `stream` is a hipStream_t (NULL = the null stream). Every call only enqueues work on it and
 *     returns; nothing synchronizes. Buffers must stay alive until the stream reaches the work.
 *   - Arguments are validated on the host before anything is enqueued; on any error nothing is
 *     enqueued and the status says why. Data preconditions (ids in [0,E), a CSR
 *     produced by moe_bucket with the same E/tile_m/mpad_max) are documented, not checked.
 *   - bf16 values are passed as their 16-bit patterns (uint16_t).
 *   - Results are deterministic: two identical calls produce bit-identical outputs (no float
 *     atomics anywhere).
 */
#ifndef MOE_MX4_H
#define MOE_MX4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,  /* NULL pointer, non-positive size, k outside [1, min(E, MOE_MAX_K)]          */
  MOE_ESHAPE = 2,  /* K % 32 != 0, odd N with SwiGLU, tile_m outside [1, MOE_MAX_TILE_M],
                      mpad_max smaller than moe_mpad_max(...), E above MOE_MAX_E            */
  MOE_EALIGN = 3,  /* weights, activations or outputs not 16-byte aligned                      */
  MOE_ELAUNCH = 4  /* the HIP runtime reported an error when the kernel was enqueued          */
} moe_status;
/* Launch errors are read with hipGetLastError() right after each launch, and the runtime's
   last-error state is cleared just before it: an error left there by an earlier, unrelated call
   of the caller's is consumed by the next entry point and not reported as its own. */

typedef enum {
  MOE_ACT_NONE = 0,       /* out = f32 [mpad_max][N]: bias + a . W^T                              */
  MOE_ACT_SWIGLU_OAI = 1, /* out = bf16 [mpad_max][N/2]: clamped SwiGLU-OAI of (gate, up) halves */
  MOE_ACT_SWIGLU_OAI_MX8 = 2 /* mx4_moe_gemm_mx8 only: the SwiGLU-OAI rows, rounded to bf16, then
                                written as MXFP8 rows (out: E4M3 [mpad_max][N/2], out_scale:
                                e8m0 [mpad_max][roundup(N/64, 16)]), bit for bit what
                                mx8_quantize makes of the bf16 rows                           */
} moe_act;

#define MOE_MAX_K 16        /* experts per token */
#define MOE_MAX_E 1024      /* experts per layer */
#define MOE_MAX_TILE_M 256  /* bucket padding granule */
#define MOE_GEMV_MAX_K 16384 /* reduction length of mx4_moe_gemv (mx4_moe_gemm has no limit) */
#define MOE_SCALE_ROW_ALIGN 16 /* bytes: scale rows of the chunked layout are padded to this */

/* Host helper of the boundary (no passage: the pages define no error reporting). Static,
   NUL-terminated description of a status code (never NULL); unknown codes get a generic text. */
const char* moe_strerror(int status);

/*
 * Host helper (no kernel). Follows PR #3579 "dasLLAMA gpt-oss arc", Metal fusion-lane commit:
 * the bucket pads every expert's run of rows to the matmul's tile granule and places the runs at
 * padded prefix bases, so the row space the CSR needs is bounded as below (the pages give no
 * formula; this is the plain bound of that layout, and the caller sizes row_tok and the GEMM
 * outputs with it).
 * Row capacity of the CSR for T tokens routed to k of E experts with padding granule tile_m:
 *   R = T*k routed rows; every non-empty expert pads its rows up to a multiple of tile_m, so at
 *   most min(E, R) experts each add at most tile_m-1 padding rows:
 *   mpad_max = roundup(R + min(E, R) * (tile_m - 1), tile_m).
 * Returns -1 for invalid arguments (T < 1, k < 1, E < 1, k > E, tile_m < 1). Host-only.
 */
int64_t moe_mpad_max(int64_t T, int k, int E, int tile_m);

/*
 * Top-k routing ([chain]: expert ids per token; [mx4]: k = 4 experts per token at gpt-oss shape).
 *   logits  f32 [T][E], row-major.
 *   ids     i32 [T][k] out: for each token, the k largest logits in descending order; equal logits
 *           are ordered by ascending expert id (-0.0 and +0.0 are equal). A NaN logit ranks below
 *           every number (-inf included), NaNs among themselves by id: the order is total, so
 *           every row, NaN rows included, yields k distinct ids in [0, E) (the pages route finite
 *           logits; this reading only makes any input safe). Every call that routes (moe_router,
 *           mx4_moe_decode, mx4_moe_decode_persistent) uses this same order.
 *   w       f32 [T][k] out: softmax over the k selected logits,
 *           w[s] = exp(l[s]-l[0]) / sum_j exp(l[j]-l[0]), evaluated in double and rounded to f32
 *           (NaN where a NaN logit is among the k).
 * Errors: MOE_EINVAL for NULL pointers, T < 1, E < 1, k < 1, k > min(E, MOE_MAX_K);
 *         MOE_ESHAPE for E > MOE_MAX_E.
 */
int moe_route_topk(const float* logits, int64_t T, int E, int k, int32_t* ids, float* w,
                   void* stream);

/*
 * Bucket / CSR of routed rows per expert with padded prefix bases ([fusion]: one workgroup per
 * expert computes its own padded-prefix base and publishes basep[e]).
 *   ids      i32 [T][k] in, each id in [0, E), distinct within a token.
 *   counts   i32 [E]   out: cnt[e] = number of (t, s) with ids[t][s] == e.
 *   basep    i32 [E+1] out: basep[0] = 0, basep[e+1] = basep[e] + roundup(cnt[e], tile_m).
 *   row_tok  i32 [mpad_max] out: row basep[e] + j holds the token of expert e's j-th routed row,
 *            rows ordered by ascending token; padding rows [basep[e]+cnt[e], basep[e+1]) and ghost
 *            rows [basep[E], mpad_max) hold -1.
 *   pos      i32 [T][k] out: the CSR row of (t, s), i.e. row_tok[pos[t][s]] == t.
 * Errors: MOE_EINVAL for NULL pointers, T < 1, k < 1, E < 1, k > min(E, MOE_MAX_K);
 *         MOE_ESHAPE for tile_m outside [1, MOE_MAX_TILE_M], E > MOE_MAX_E, or
 *         mpad_max < moe_mpad_max(T, k, E, tile_m).
 */
int moe_bucket(const int32_t* ids, int64_t T, int k, int E, int tile_m, int64_t mpad_max,
               int32_t* counts, int32_t* basep, int32_t* row_tok, int32_t* pos, void* stream);

/*
 * A stack of E MXFP4 expert matrices W[e] of N rows by K columns ([mx4]).
 * Element values: decoded element = e2m1(code) * 2^(scale - 127) as an fp32 value (+-inf if it
 * exceeds the fp32 range; NaN for scale byte 255), e2m1 = {0, .5, 1, 1.5, 2, 3, 4, 6} with bit 3
 * the sign; element 2i of a row is the LOW nibble of byte i of the row, element 2i+1 the HIGH.
 * For the gate_up projection N = 2*ffn, rows [0, ffn) are the gate and rows [ffn, 2*ffn) the up
 * projection; for the down projection N = dim.
 *
 * Two byte layouts of the same stack (KB = K/32 blocks per row; a block = 16 nibble bytes +
 * 1 scale byte):
 *   checkpoint layout (row-major, as stored by gpt-oss checkpoints)
 *     q [E][N][K/2] bytes, s [E][N][KB] bytes.
 *   chunked layout (what the projections read):
 *     nibbles: each expert's K is cut into chunks of 4 blocks, C = ceil(KB/4) chunks, chunk c
 *       holding blocks [4c, 4c + w_c), w_c = min(4, KB - 4c), stored chunk after chunk with all
 *       N rows of a chunk together: the 16 nibble bytes of block (e, n, kb) start at byte
 *       16 * (e*N*KB + (kb/4)*N*4 + n*w_c + (kb%4)). Same size as the checkpoint's q. Every
 *       16 consecutive rows of a chunk are one contiguous run of 16*w_c*16 bytes, which is what
 *       one wavefront of the projection kernels reads per load instruction.
 *     scales: each row's KB scale bytes are cut into G = ceil(KB/16) groups of 16 (the scales
 *       of 4 chunks), stored group after group with all N rows of a group together: the scale
 *       of block (e, n, kb) is byte 16 * ((e*G + kb/16)*N + n) + kb%16, and the bytes past KB
 *       in the last group are 0. Size E*N*SP bytes, SP = 16*G = roundup(KB, 16). Every 16
 *       consecutive rows of a group are one contiguous 256-byte run, which one wavefront reads
 *       with one load.
 * mx4_experts describes a stack in the CHUNKED layout. The descriptor itself is a HOST struct;
 * q, s and bias are device pointers; bias is f32 [E][N] or NULL.
 */
typedef struct {
  const uint8_t* q;
  const uint8_t* s;
  const float* bias;
  int E;
  int N;
  int K;
} mx4_experts;

/*
 * Repack an expert stack from the checkpoint layout to the chunked layout (a byte permutation
 * plus the zero padding of the last scale group, run once when the weights are loaded). q_src/s_src in the
 * checkpoint layout (E*N*K/2 and E*N*K/32 bytes); q_dst (E*N*K/2 bytes) and s_dst
 * (E*N*roundup(K/32, 16) bytes) receive the chunked layout; no buffer may overlap another.
 * Errors: MOE_EINVAL for NULL pointers or E/N < 1; MOE_ESHAPE for K < 32 or K % 32 != 0;
 *         MOE_EALIGN for q_src, q_dst or s_dst not 16-byte aligned; MOE_ELAUNCH.
 */
int mx4_pack_experts(const uint8_t* q_src, const uint8_t* s_src, int E, int N, int K,
                     uint8_t* q_dst, uint8_t* s_dst, void* stream);

/*
 * Routed-expert MXFP4 projection, bias-seeded, with an optional fused SwiGLU-OAI epilogue
 * ([fusion]: accumulators start from the expert's bias row, the SwiGLU-OAI epilogue skips ghost
 * rows; [chain]: gate and up rows + bias + activation in one stage).
 * For every expert e and every live CSR row r in [basep[e], basep[e] + counts[e]):
 *   act row   x = a[a_row[r]] if a_row != NULL, else a[r]          (bf16, K elements)
 *   g[n]      = bias[e][n] + sum_i x[i] * W[e][n][i]   (fp32 accumulation), n in [0, N)
 *   MOE_ACT_NONE:        out f32  [mpad_max][N]:   out[r][n] = g[n]
 *   MOE_ACT_SWIGLU_OAI:  out bf16 [mpad_max][N/2]: with F = N/2, for j in [0, F):
 *        gc = min(g[j], limit), uc = clamp(g[F+j], -limit, limit),
 *        out[r][j] = bf16_rne( gc * sigmoid(alpha * gc) * (uc + 1) )
 * Rows that are padding or ghost (not live) are left UNWRITTEN; empty experts do no work.
 *   a         bf16 [a_rows][K] activations, row-major.
 *   a_row     i32 [mpad_max] or NULL (the row_tok array of moe_bucket for the gate_up step;
 *             NULL for the down step, whose input rows are already in CSR order). Every live
 *             row's a_row entry must be in [0, a_rows); with a_row == NULL a_rows >= mpad_max.
 *   counts, basep: from moe_bucket (same E, tile_m, mpad_max).
 * mx4_moe_gemv and mx4_moe_gemm compute the same function with different kernels, both
 * dequantizing MXFP4 to bf16 in registers for bf16 MFMA with fp32 accumulation: the GEMV keeps
 * a whole K segment of each wavefront's weights in flight and takes up to 16 routed rows per
 * pass (decode, a handful of rows per expert), the GEMM runs over all of an expert's rows per
 * workgroup in 16-row tiles (prefill, tens to hundreds of rows per expert). Their results agree
 * within fp32 summation order, not bit-for-bit.
 * Errors: MOE_EINVAL for NULL a/w/q/s/counts/basep/out, a_rows < 1, E/N < 1, mpad_max < 1,
 *         unknown act; MOE_ESHAPE for K < 32 or K % 32 != 0 (mx4_moe_gemv also for
 *         K > MOE_GEMV_MAX_K), odd N with MOE_ACT_SWIGLU_OAI,
 *         tile_m outside [1, MOE_MAX_TILE_M], E > MOE_MAX_E, a_row == NULL with
 *         a_rows < mpad_max; MOE_EALIGN for q, a or out not 16-byte aligned;
 *         MOE_ELAUNCH if the runtime rejects the launch.
 */
int mx4_moe_gemv(const uint16_t* a, const int32_t* a_row, int64_t a_rows, const mx4_experts* w,
                 const int32_t* counts, const int32_t* basep, int tile_m, int64_t mpad_max,
                 int act, float alpha, float limit, void* out, void* stream);

int mx4_moe_gemm(const uint16_t* a, const int32_t* a_row, int64_t a_rows, const mx4_experts* w,
                 const int32_t* counts, const int32_t* basep, int tile_m, int64_t mpad_max,
                 int act, float alpha, float limit, void* out, void* stream);

#define MOE_ROUTER_MAX_ROUTED 16384  /* T*k of one moe_router call */
#define MOE_ROUTER_WS_WORDS 67584    /* u32 workspace words of moe_router */

/*
 * The router projection and the routing front of the chain in one launch: the step before the
 * routed chain ([ext, gpt-oss]: the router is a linear layer with bias) fused with top-k and
 * the bucket pass ([chain]: per-token expert ids in slot order; [fusion]: the padded-prefix
 * bases computed inside the bucket pass, the CSR unchanged).
 *   logits[t][e] = b_r[e] + sum_d x[t][d] * W_r[e][d]   bf16 products, fp32 accumulation
 *   ids, w      = moe_route_topk of those fp32 logits (bit for bit the same decisions)
 *   counts, basep, row_tok, pos = moe_bucket of those ids with tile_m and mpad_max
 *   x     bf16 [T][D];  w_r bf16 [E][D];  b_r f32 [E] or NULL.
 *   logits f32 [T][E] out, or NULL (then not written).
 *   ws    u32 [MOE_ROUTER_WS_WORDS] device workspace owned by the caller: zero before the first
 *         call, then left to the library. Word 0 and words 64..1087 are completion counters
 *         that every call leaves zero; the rest holds the last call's partial logits or top-k
 *         candidates. Calls that can run concurrently need distinct workspaces.
 * Work split: for T <= 16 and E <= 256 the reduction over D is split over up to 48 workgroups,
 * whose partial logits are summed in a fixed order (results are deterministic; they differ from
 * the one-workgroup sum only by fp32 association). Otherwise a workgroup takes 16 tokens; for
 * E >= 64 and at most one round of pairs over the CUs, a pair of workgroups takes them, each
 * with half of the experts, and the later of the pair merges the two halves' top-k candidates
 * (the same picks as one pass). The workgroup that finishes last builds the CSR (from
 * per-group histograms that fit 64 KB of LDS, else by sweeping all ids per expert), found by
 * counting on word 0; no workgroup waits for another.
 * Errors: MOE_EINVAL for NULL pointers (other than b_r, logits), T, D or E < 1, k < 1,
 *         k > min(E, MOE_MAX_K); MOE_ESHAPE for D % 32 != 0, T*k > MOE_ROUTER_MAX_ROUTED,
 *         E > MOE_MAX_E, tile_m outside [1, MOE_MAX_TILE_M], mpad_max < moe_mpad_max(T, k, E,
 *         tile_m), x or W_r of 2 GB or more; MOE_EALIGN for x or w_r not 16-byte aligned or ws
 *         not 4-byte aligned; MOE_ELAUNCH.
 */
int moe_router(const uint16_t* x, const uint16_t* w_r, const float* b_r, int64_t T, int D,
               int E, int k, int tile_m, int64_t mpad_max, float* logits, int32_t* ids, float* w,
               int32_t* counts, int32_t* basep, int32_t* row_tok, int32_t* pos, uint32_t* ws,
               void* stream);

/*
 * MXFP8 activations: the projections on the MX-scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4,
 * E2M1 weights x E4M3 activations, each 32-value block carrying its own e8m0 scale). The pages
 * quantize only the weights: this variant and every fact of its format come from outside them,
 * the OCP 8-bit floating point spec (E4M3) and the OCP Microscaling v1.0 spec (conversion of a
 * 32-value block to one shared e8m0 scale plus 32 elements). It changes the numerics: the
 * activations are rounded to 4 significant bits before the product.
 *
 * MXFP8 row layout: row r of K values has its K E4M3 bytes at q + r*K (element i = byte i) and
 * its K/32 e8m0 bytes at s + r*SP, SP = roundup(K/32, 16); the SP - K/32 padding bytes are 0.
 *
 * mx8_quantize: the OCP MX conversion of bf16 rows, exactly (bit for bit) as follows. For each
 * block of 32 consecutive values with largest magnitude m: the shared exponent is
 * X = floor(log2(m)) - 8 (8 = exponent of E4M3's largest normal), clamped to [-127, 127];
 * a block of zeros (or of magnitudes below 2^-126) takes X = -127; its scale byte is X + 127.
 * Each element is v / 2^X rounded to the nearest E4M3 value, ties to the even mantissa,
 * magnitudes beyond 448 saturating to 448 (never NaN); the sign bit is v's, so -0 and negatives
 * that round to zero give byte 0x80.
 *   a     bf16 [rows][K] row-major, finite values (not checked).
 *   live  i32 [rows] or NULL: rows with live[r] < 0 are skipped (q and s rows left unwritten),
 *         e.g. the row_tok array of moe_bucket when quantizing h, whose padding and ghost rows
 *         hold nothing.
 *   q     u8 [rows][K] out; s u8 [rows][SP] out (padding bytes written 0).
 * Errors: MOE_EINVAL for NULL a/q/s or rows < 1; MOE_ESHAPE for K < 32, K % 32 != 0 or
 *         rows * K >= 2^31; MOE_EALIGN for a, q or s not 16-byte aligned; MOE_ELAUNCH.
 *
 * mx4_moe_gemm_mx8: the function of mx4_moe_gemm with activation row x = the MXFP8 row
 * a_row[r] (or r) of (aq, as) in place of a bf16 row: g[n] = bias[e][n] + sum_i x[i]*W[e][n][i]
 * with x[i] = e4m3(aq[..][i]) * 2^(as[..][i/32] - 127), accumulated in fp32 by the MFMA
 * (products are exact; the hardware's sum over a 128-value step is not rounded like a chain of
 * fp32 additions but stays within the same error bound, |error| <= 1e-3 * sum |x_i W_i|).
 * Arguments, row semantics, epilogue (MOE_ACT_NONE / MOE_ACT_SWIGLU_OAI) and outputs as
 * mx4_moe_gemm; a_rows counts MXFP8 rows. MOE_ACT_SWIGLU_OAI_MX8 writes the SwiGLU-OAI rows
 * directly as MXFP8 rows (out: E4M3 bytes, out_scale: e8m0 rows with zero padding), the input
 * format of the down projection, so the bf16 rows never leave the chip; out_scale is unused
 * (may be NULL) otherwise.
 * Errors: as mx4_moe_gemm (aq in place of a, also NULL as), plus MOE_ESHAPE for
 *         K > MOE_MX8_GEMM_MAX_K, MOE_EINVAL for MOE_ACT_SWIGLU_OAI_MX8 with out_scale NULL,
 *         MOE_ESHAPE for it with N % 64 != 0, MOE_EALIGN for as or out_scale not 16-byte
 *         aligned.
 */
#define MOE_MX8_GEMM_MAX_K 4096  /* reduction length of mx4_moe_gemm_mx8 (LDS scale staging) */

int mx8_quantize(const uint16_t* a, const int32_t* live, int64_t rows, int K, uint8_t* q,
                 uint8_t* s, void* stream);

int mx4_moe_gemm_mx8(const uint8_t* aq, const uint8_t* as, const int32_t* a_row, int64_t a_rows,
                     const mx4_experts* w, const int32_t* counts, const int32_t* basep, int tile_m,
                     int64_t mpad_max, int act, float alpha, float limit, void* out,
                     uint8_t* out_scale, void* stream);

#define MOE_DECODE_MAX_T 16  /* tokens per mx4_moe_decode call */
#define MOE_DECODE_MAX_K 8   /* experts per token in mx4_moe_decode */

/*
 * The whole routed chain of a few tokens in two launches ([chain]: stage 1 = gate and up rows +
 * bias + activation, stage 2 = down rows + bias and the routing-weighted sum in slot order;
 * [fusion]: bias-seeded accumulators, per-expert padded-prefix bases). Computes exactly what
 * moe_route_topk, moe_bucket (tile_m = 1), mx4_moe_gemv with MOE_ACT_SWIGLU_OAI, mx4_moe_gemv
 * with MOE_ACT_NONE and moe_combine compute, except that h and d are indexed by ROUTED ROW
 * rho = t*k + s (token t, slot s) instead of by CSR row:
 *   ids, w      i32/f32 [T][k]  routing (as moe_route_topk)
 *   counts [E], basep [E+1], row_tok [T*k], pos [T][k]: the CSR with tile_m = 1 (as moe_bucket;
 *               mpad = T*k, no padding rows)
 *   h     bf16 [T*k][F]  h[rho] = SwiGLU-OAI(gate_up projection of x[t] by expert ids[t][s])
 *   d     f32  [T*k][D]  d[rho] = down projection of h[rho] by that expert, bias included; may be
 *                        NULL (then never written: the combine happens on chip)
 *   y     f32  [T][D]    y[t][n] = sum over s in slot order of w[t][s] * d[t*k+s][n]
 *   logits f32 [T][E], x bf16 [T][D]; w_gu: E experts of [2F][D] (gate rows [0,F), up rows
 *   [F,2F)), w_dn: E experts of [D][F], both in the chunked layout of mx4_pack_experts.
 * Each pick streams its expert's weights once, so an expert picked by several of the T tokens
 * is read several times: for more than a few tokens the CSR calls are the cheaper path.
 * Errors: MOE_EINVAL for NULL pointers (other than d), T < 1, E < 1, k < 1, k > min(E,
 *         MOE_MAX_K); MOE_ESHAPE for T > MOE_DECODE_MAX_T, k > MOE_DECODE_MAX_K, E > MOE_MAX_E,
 *         w_gu / w_dn with another E, D or F not a positive multiple of 32, w_dn not [D][F],
 *         activation rows too long for LDS (k*F*2 bytes above ~55 KB); MOE_EALIGN for x, h or the
 *         weight arrays not 16-byte aligned, logits, d or y not 4-byte aligned; MOE_ELAUNCH if
 *         the runtime rejects a launch.
 */
int mx4_moe_decode(const float* logits, const uint16_t* x, int64_t T, int E, int k,
                   const mx4_experts* w_gu, const mx4_experts* w_dn, float alpha, float limit,
                   int32_t* ids, float* w, int32_t* counts, int32_t* basep, int32_t* row_tok,
                   int32_t* pos, uint16_t* h, float* d, float* y, void* stream);

#define MOE_DECODE_WS_WORDS 544  /* u32 workspace words of mx4_moe_decode_persistent */

/*
 * The same chain as mx4_moe_decode in ONE launch ([chain]'s two stages without the launch
 * boundary between them), built so that every weight byte of the layer is in flight as soon as
 * the routing is known: a grid of one workgroup per CU (all resident at once) in which every
 * workgroup routes the tokens itself, then every wavefront issues the loads of a whole work
 * item (16 weight rows of one pick over half the reduction): gate_up items, and the items of
 * the workgroup's down tiles (16 output rows of a token, every slot), which wait, holding their
 * weights in registers, until every workgroup has stored its h rows; d and y are then formed on
 * chip in slot order. Outputs and layouts are those of mx4_moe_decode; routing and the CSR are
 * identical bit for bit, h, d and y within the same tolerances (the reduction is split in two
 * halves here, so fp32 sums may associate differently; at a given grid the results are
 * deterministic).
 *   ws    u32 [MOE_DECODE_WS_WORDS] device workspace owned by the caller: zero before the first
 *         call, then left alone (the library keeps its completion counters and a call epoch
 *         there). Calls that can run concurrently need distinct workspaces. Word 3 is an error
 *         flag the call sets (and never clears) if a wait ran past its bound (about a second);
 *         the outputs of that call are then invalid. This cannot happen while the grid is
 *         resident as sized here.
 *   max_workgroups  0, or a cap on the grid (at least 1) for callers sharing the GPU.
 * Shapes the one-launch kernel does not take (2k > 8, E > 64, F % 8 != 0, D or F above 3072,
 * or LDS beyond 64 KB for the grid) run as the two launches of mx4_moe_decode instead; ws is
 * then untouched.
 * Errors: those of mx4_moe_decode, plus MOE_EINVAL for ws == NULL or max_workgroups < 0,
 *         MOE_EALIGN for ws not 4-byte aligned, MOE_ELAUNCH if the occupancy query fails.
 */
int mx4_moe_decode_persistent(const float* logits, const uint16_t* x, int64_t T, int E, int k,
                              const mx4_experts* w_gu, const mx4_experts* w_dn, float alpha,
                              float limit, int32_t* ids, float* w, int32_t* counts,
                              int32_t* basep, int32_t* row_tok, int32_t* pos, uint16_t* h,
                              float* d, float* y, uint32_t* ws, int max_workgroups,
                              void* stream);

/*
 * mx4_moe_decode_persistent for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no workspace argument.
 * The workspace is the library's own, a file-scope device array of MOE_DECODE_WS_WORDS u32 words
 * (2176 bytes) that every GPU the library runs on holds until the process ends. Nothing is
 * allocated: a call that runs the one-launch kernel first enqueues a one-workgroup kernel that
 * zeroes that array (a kernel, not a memset, so the call can be captured), then the layer kernel;
 * the shapes the one-launch kernel does not take run as the two launches of mx4_moe_decode,
 * which use no workspace. The array has the same size at every shape (it holds counters, not
 * data); shapes beyond the limits of mx4_moe_decode_persistent are rejected with its errors.
 * Every call on a GPU shares that GPU's array: calls that can overlap on one GPU (other streams,
 * other threads) race, and only one may be in flight per GPU at a time. The workspace's error
 * flag (a wait past its bound) is not reported by this variant.
 * Arguments and outputs are those of mx4_moe_decode_persistent without ws; for equal arguments
 * the outputs are bit-identical to it.
 * Errors: those of mx4_moe_decode_persistent other than the ws ones, plus MOE_ELAUNCH if the
 *         array's device address cannot be obtained.
 */
int mx4_moe_decode_persistent_static(const float* logits, const uint16_t* x, int64_t T, int E,
                                     int k, const mx4_experts* w_gu, const mx4_experts* w_dn,
                                     float alpha, float limit, int32_t* ids, float* w,
                                     int32_t* counts, int32_t* basep, int32_t* row_tok,
                                     int32_t* pos, uint16_t* h, float* d, float* y,
                                     int max_workgroups, void* stream);

/*
 * Router-weighted combine ([chain]: routing-weighted sum of the expert rows in slot order).
 *   y[t][n] = sum_{s=0..k-1} w[t][s] * d[pos[t][s]][n], accumulated in fp32 in slot order.
 *   d    f32 [d_rows][D], the down projection's output in CSR row order (bias included).
 *   pos  i32 [T][k] from moe_bucket; every entry in [0, d_rows).
 *   w    f32 [T][k] from moe_route_topk.
 *   y    f32 [T][D] out, fully written.
 * Errors: MOE_EINVAL for NULL pointers, T < 1, k < 1 or k > MOE_MAX_K, D < 1, d_rows < 1;
 *         MOE_EALIGN for d or y not 4-byte aligned.
 */
int moe_combine(const float* d, int64_t d_rows, const int32_t* pos, const float* w, int64_t T,
                int k, int D, float* y, void* stream);

#define MOE_TIMING_MAX 64   /* launches one moe_timing_arm can time */

/*
 * Kernel timing, for measurement. After moe_timing_arm(n), the next n kernel launches made by
 * any call of this library (in launch order, on whatever stream) are launched with a pair of
 * HIP events that the runtime stamps at the kernel's own start and end (hipExtLaunchKernel),
 * i.e. the kernel execution interval a kernel trace reports, without the dispatch gaps around
 * it. moe_timing_read(ms, n) waits for the first n timed launches since the arm and writes
 * their durations in milliseconds. moe_timing_arm(0) disarms. The event pairs are created on
 * the current device at the first arm and kept until the process ends (the one exception to
 * "keeps no state"). Not thread-safe; never arm while a stream is being captured into a graph.
 * Errors: MOE_EINVAL for n outside [0, MOE_TIMING_MAX] or ms == NULL; MOE_ESHAPE for reading
 *         more launches than were timed; MOE_ELAUNCH if the runtime fails to create or read an
 *         event.
 */
int moe_timing_arm(int n);
int moe_timing_read(float* ms, int n);

/*
 * Attained-peak probes, for measurement only (they are not steps of the chain): the rates a
 * plain kernel reaches on this GPU, reported beside the published peaks.
 *   moe_probe_read: reads every byte of src (device, 16-byte aligned, bytes a multiple of 16)
 *     once with nontemporal 16-byte loads, 8 in flight per lane, grid-stride over `workgroups` workgroups of
 *     256 threads. Algorithmic bytes = bytes. sink (device u32) is written only if the xor of
 *     every word equals 0x9E3779B9 (a guard that keeps the loads; its value means nothing).
 *   moe_probe_mfma_bf16: `workgroups` workgroups of 4 wavefronts, each wavefront issuing
 *     iters x 4 independent v_mfma_f32_32x32x16_bf16 (32*32*16*2 = 32768 flops each), so
 *     flops = workgroups * 4 * iters * 4 * 32768. sink (device f32) is a guard like the read's.
 * Errors: MOE_EINVAL for NULL pointers, bytes < 16, workgroups < 1 or iters < 1; MOE_EALIGN for
 *         src or bytes not 16-byte aligned; MOE_ELAUNCH.
 */
int moe_probe_read(const void* src, int64_t bytes, uint32_t* sink, int workgroups, void* stream);
int moe_probe_mfma_bf16(int workgroups, int iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MX4_H */
