// C ABI entry points of the expert projections: host-side argument checks, then the launch.
// Every check runs before anything is enqueued; on failure nothing is enqueued.
#include "common.hpp"

int moe_launch_gemv(const uint16_t* a, const int32_t* a_row, int64_t a_rows, const mx4_experts* w,
                    const int32_t* counts, const int32_t* basep, int tile_m, int64_t mpad_max,
                    int act, float alpha, float limit, void* out, hipStream_t stream);
int moe_launch_gemm(const uint16_t* a, const int32_t* a_row, int64_t a_rows, const mx4_experts* w,
                    const int32_t* counts, const int32_t* basep, int tile_m, int64_t mpad_max,
                    int act, float alpha, float limit, void* out, hipStream_t stream);

int moe_launch_gemm_mx8(const uint8_t* aq, const uint8_t* as, const int32_t* a_row,
                        int64_t a_rows, const mx4_experts* w, const int32_t* counts,
                        const int32_t* basep, int tile_m, int64_t mpad_max, int act, float alpha,
                        float limit, void* out, uint8_t* out_scale, hipStream_t stream);

namespace {

int check_projection(const void* a, const int32_t* a_row, int64_t a_rows,
                     const mx4_experts* w, const int32_t* counts, const int32_t* basep,
                     int tile_m, int64_t mpad_max, int act, void* out) {
  if (!a || !w || !w->q || !w->s || !counts || !basep || !out) return MOE_EINVAL;
  if (a_rows < 1 || w->E < 1 || w->N < 1 || mpad_max < 1) return MOE_EINVAL;
  if (act != MOE_ACT_NONE && act != MOE_ACT_SWIGLU_OAI) return MOE_EINVAL;
  if (w->K < 32 || (w->K % 32) != 0) return MOE_ESHAPE;
  if (act == MOE_ACT_SWIGLU_OAI && (w->N % 2) != 0) return MOE_ESHAPE;
  if (tile_m < 1 || tile_m > MOE_MAX_TILE_M || w->E > MOE_MAX_E) return MOE_ESHAPE;
  if (mpad_max > 0x7FFFFFFFLL) return MOE_ESHAPE;
  if (!a_row && a_rows < mpad_max) return MOE_ESHAPE;
  if ((((uintptr_t)w->q) & 15) || (((uintptr_t)a) & 15) || (((uintptr_t)out) & 15))
    return MOE_EALIGN;
  return MOE_OK;
}

}  // namespace

extern "C" const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (NULL pointer, non-positive size, or k/act out of range)";
    case MOE_ESHAPE: return "unsupported shape (K % 32, odd N with SwiGLU, tile_m, E, or mpad_max too small)";
    case MOE_EALIGN: return "misaligned pointer (weights, activations and outputs need 16-byte alignment)";
    case MOE_ELAUNCH: return "the HIP runtime rejected the kernel launch";
    default: return "unknown status";
  }
}

extern "C" int mx4_moe_gemv(const uint16_t* a, const int32_t* a_row, int64_t a_rows,
                            const mx4_experts* w, const int32_t* counts, const int32_t* basep,
                            int tile_m, int64_t mpad_max, int act, float alpha, float limit,
                            void* out, void* stream) {
  const int st = check_projection(a, a_row, a_rows, w, counts, basep, tile_m, mpad_max, act, out);
  if (st != MOE_OK) return st;
  if (a_rows > 0x7FFFFFFFLL || w->K > MOE_GEMV_MAX_K) return MOE_ESHAPE;
  return moe_launch_gemv(a, a_row, a_rows, w, counts, basep, tile_m, mpad_max, act, alpha, limit, out,
                         (hipStream_t)stream);
}

extern "C" int mx4_moe_gemm(const uint16_t* a, const int32_t* a_row, int64_t a_rows,
                            const mx4_experts* w, const int32_t* counts, const int32_t* basep,
                            int tile_m, int64_t mpad_max, int act, float alpha, float limit,
                            void* out, void* stream) {
  const int st = check_projection(a, a_row, a_rows, w, counts, basep, tile_m, mpad_max, act, out);
  if (st != MOE_OK) return st;
  return moe_launch_gemm(a, a_row, a_rows, w, counts, basep, tile_m, mpad_max, act, alpha, limit, out,
                         (hipStream_t)stream);
}

extern "C" int mx4_moe_gemm_mx8(const uint8_t* aq, const uint8_t* as, const int32_t* a_row,
                                int64_t a_rows, const mx4_experts* w, const int32_t* counts,
                                const int32_t* basep, int tile_m, int64_t mpad_max, int act,
                                float alpha, float limit, void* out, uint8_t* out_scale,
                                void* stream) {
  if (!as) return MOE_EINVAL;
  const bool q_out = act == MOE_ACT_SWIGLU_OAI_MX8;
  if (q_out && !out_scale) return MOE_EINVAL;
  // the MXFP8 output takes the SwiGLU shape checks
  const int st = check_projection(aq, a_row, a_rows, w, counts, basep, tile_m, mpad_max,
                                  q_out ? MOE_ACT_SWIGLU_OAI : act, out);
  if (st != MOE_OK) return st;
  if (w->K > MOE_MX8_GEMM_MAX_K || (q_out && w->N % 64 != 0)) return MOE_ESHAPE;
  if ((((uintptr_t)as) & 15) || (q_out && (((uintptr_t)out_scale) & 15))) return MOE_EALIGN;
  return moe_launch_gemm_mx8(aq, as, a_row, a_rows, w, counts, basep, tile_m, mpad_max, act, alpha,
                             limit, out, out_scale, (hipStream_t)stream);
}
