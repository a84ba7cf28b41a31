// C ABI of libmoe: argument checks on the host, then kernel launches.
// Every check runs before any HIP call, so a rejected call enqueues nothing.
#include <limits.h>

#include <algorithm>

#include "moe_internal.h"

using moe::WsLayout;

namespace {

// Shape checks shared by every entry point.
moe_status check_shape(const moe_shape& s) {
  if (s.T <= 0 || s.H <= 0 || s.E <= 0 || s.k <= 0 || s.I <= 0) return MOE_EINVAL;
  if (s.k > s.E || s.E > 1024) return MOE_EINVAL;
  if (static_cast<int64_t>(s.T) * s.k >= (static_cast<int64_t>(1) << 31)) return MOE_EINVAL;
  if (s.dtype != MOE_F32 && s.dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (s.H % 64 != 0 || s.I % 64 != 0) return MOE_EUNSUPPORTED;
  // Element offsets inside one expert's weights and one row block stay int32.
  if (static_cast<int64_t>(s.E) * s.I * s.H >= (static_cast<int64_t>(1) << 31)) return MOE_EUNSUPPORTED;
  // The weight-gradient tile plan counts work (tiles x 32-row k-steps) in int32.
  const int64_t tiles = static_cast<int64_t>((2 * s.I + 255) / 256) * ((s.H + 255) / 256);
  if (tiles * (static_cast<int64_t>(s.T) * s.k / 32 + s.E) >= (static_cast<int64_t>(1) << 30)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

template <class... P>
bool any_null(P... p) {
  return ((p == nullptr) || ...);
}

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// x read through row tokens is addressed with 32-bit byte offsets.
bool gathered_x_fits(const moe_shape& s) {
  return static_cast<int64_t>(s.T) * s.H * (s.dtype == MOE_BF16 ? 2 : 4) < (static_cast<int64_t>(1) << 31);
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(moe_shape s) {
  if (check_shape(s) != MOE_OK) return 0;
  return moe::ws_layout(s).total;
}

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: shape or dtype not supported";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP launch failed";
  }
  return "unknown moe_status";
}

moe_status moe_route(moe_shape s, const void* x, const void* w_router, const float* logit_bias, float* logits,
                     int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(x, w_router, logits, topk_idx, topk_w)) return MOE_EINVAL;
  return from_hip(moe::launch_route(s, x, w_router, logit_bias, logits, topk_idx, topk_w, stream));
}

moe_status moe_permute(moe_shape s, const int32_t* topk_idx, const void* x, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_to_flat, int32_t* flat_to_sorted, void* x_perm, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(topk_idx, x, counts, offsets, sorted_to_flat, flat_to_sorted, x_perm, ws)) return MOE_EINVAL;
  if (ws_bytes < moe::ws_layout(s).total) return MOE_EWORKSPACE;
  return from_hip(moe::launch_permute(s, topk_idx, x, counts, offsets, sorted_to_flat, flat_to_sorted, x_perm, ws,
                                      stream));
}

moe_status moe_gemm_gate_up(moe_shape s, const void* x_perm, const int32_t* offsets, const void* w_gate,
                            const void* w_up, void* g, void* u, void* a, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(x_perm, offsets, w_gate, w_up, g, u, a)) return MOE_EINVAL;
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = x_perm;
  ga.b0 = w_gate;
  ga.b1 = w_up;
  ga.out0 = g;
  ga.out1 = u;
  ga.out2 = a;
  return from_hip(moe::launch_gemm(moe::GEMM_GATEUP, s, ga, stream));
}

moe_status moe_gemm_down(moe_shape s, const void* a, const int32_t* offsets, const void* w_down, void* o_perm,
                         hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(a, offsets, w_down, o_perm)) return MOE_EINVAL;
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = a;
  ga.b0 = w_down;
  ga.out0 = o_perm;
  return from_hip(moe::launch_gemm(moe::GEMM_DOWN, s, ga, stream));
}

moe_status moe_gemm_down_dgrad(moe_shape s, const void* do_perm, const int32_t* offsets, const void* w_down,
                               const void* g, const void* u, void* dgu, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(do_perm, offsets, w_down, g, u, dgu)) return MOE_EINVAL;
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = do_perm;
  ga.b0 = w_down;
  ga.g_in = g;
  ga.u_in = u;
  ga.out0 = dgu;
  return from_hip(moe::launch_gemm(moe::GEMM_DGRAD_DOWN, s, ga, stream));
}

moe_status moe_gemm_down_wgrad(moe_shape s, const void* do_perm, const void* a, const int32_t* offsets,
                               float* dw_down, int accumulate_dw, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(do_perm, a, offsets, dw_down, ws)) return MOE_EINVAL;
  if (accumulate_dw != 0 && accumulate_dw != 1) return MOE_EINVAL;
  const WsLayout l = moe::ws_layout(s);
  if (ws_bytes < l.total) return MOE_EWORKSPACE;
  moe::GemmArgs ga{};
  ga.part = reinterpret_cast<float*>(static_cast<char*>(ws) + l.part_off);
  ga.offsets = offsets;
  ga.a = do_perm;
  ga.b0 = a;
  ga.dw0 = dw_down;
  ga.accumulate = accumulate_dw;
  return from_hip(moe::launch_gemm(moe::GEMM_WGRAD_DOWN, s, ga, stream));
}

moe_status moe_gemm_gate_up_dgrad(moe_shape s, const void* dgu, const int32_t* offsets, const void* w_gate,
                                  const void* w_up, void* dx_perm, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(dgu, offsets, w_gate, w_up, dx_perm)) return MOE_EINVAL;
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = dgu;
  ga.b0 = w_gate;
  ga.b1 = w_up;
  ga.out0 = dx_perm;
  return from_hip(moe::launch_gemm(moe::GEMM_DGRAD_GATEUP, s, ga, stream));
}

moe_status moe_gemm_gate_up_wgrad(moe_shape s, const void* dgu, const void* x_perm, const int32_t* offsets,
                                  float* dw_gate, float* dw_up, int accumulate_dw, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(dgu, x_perm, offsets, dw_gate, dw_up, ws)) return MOE_EINVAL;
  if (accumulate_dw != 0 && accumulate_dw != 1) return MOE_EINVAL;
  const WsLayout l = moe::ws_layout(s);
  if (ws_bytes < l.total) return MOE_EWORKSPACE;
  moe::GemmArgs ga{};
  ga.part = reinterpret_cast<float*>(static_cast<char*>(ws) + l.part_off);
  ga.offsets = offsets;
  ga.a = dgu;
  ga.b0 = x_perm;
  ga.dw0 = dw_gate;
  ga.dw1 = dw_up;
  ga.accumulate = accumulate_dw;
  return from_hip(moe::launch_gemm(moe::GEMM_WGRAD_GATEUP, s, ga, stream));
}

moe_status moe_grouped_gemm_fwd(moe_shape s, const void* x_perm, const int32_t* offsets, const void* w_gate,
                                const void* w_up, const void* w_down, void* g, void* u, void* a, void* o_perm,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(x_perm, offsets, w_gate, w_up, w_down, g, u, a, o_perm)) return MOE_EINVAL;
  st = moe_gemm_gate_up(s, x_perm, offsets, w_gate, w_up, g, u, a, stream);
  if (st != MOE_OK) return st;
  return moe_gemm_down(s, a, offsets, w_down, o_perm, stream);
}

moe_status moe_permute_fused(moe_shape s, const int32_t* topk_idx, const float* topk_w, int32_t* counts,
                             int32_t* offsets, int32_t* sorted_to_flat, int32_t* flat_to_sorted, int32_t* row_token,
                             float* row_weight, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(topk_idx, topk_w, counts, offsets, sorted_to_flat, flat_to_sorted, row_token, row_weight, ws))
    return MOE_EINVAL;
  if (ws_bytes < moe::ws_layout(s).total) return MOE_EWORKSPACE;
  return from_hip(moe::launch_permute_fused(s, topk_idx, topk_w, counts, offsets, sorted_to_flat, flat_to_sorted,
                                            row_token, row_weight, ws, stream));
}

moe_status moe_gemm_gate_up_gathered(moe_shape s, const void* x, const int32_t* row_token, const int32_t* offsets,
                                     const void* w_gate, const void* w_up, void* g, void* u, void* a,
                                     hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(x, row_token, offsets, w_gate, w_up, a)) return MOE_EINVAL;
  if ((g == nullptr) != (u == nullptr)) return MOE_EINVAL;
  // x is addressed with 32-bit byte offsets.
  if (static_cast<int64_t>(s.T) * s.H * (s.dtype == MOE_BF16 ? 2 : 4) >= (static_cast<int64_t>(1) << 31))
    return MOE_EUNSUPPORTED;
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = x;
  ga.row_token = row_token;
  ga.b0 = w_gate;
  ga.b1 = w_up;
  ga.out0 = g;
  ga.out1 = u;
  ga.out2 = a;
  return from_hip(moe::launch_gemm(moe::GEMM_GATEUP, s, ga, stream));
}

moe_status moe_gemm_gate_up_wgrad_gathered(moe_shape s, const void* dgu, const void* x, const int32_t* row_token,
                                           const int32_t* offsets, float* dw_gate, float* dw_up, int accumulate_dw,
                                           void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(dgu, x, row_token, offsets, dw_gate, dw_up, ws)) return MOE_EINVAL;
  if (accumulate_dw != 0 && accumulate_dw != 1) return MOE_EINVAL;
  const WsLayout l = moe::ws_layout(s);
  if (ws_bytes < l.total) return MOE_EWORKSPACE;
  // x and row_token are addressed with 32-bit byte offsets.
  if (static_cast<int64_t>(s.T) * s.H * (s.dtype == MOE_BF16 ? 2 : 4) >= (static_cast<int64_t>(1) << 31) ||
      4 * (static_cast<int64_t>(s.T) * s.k + 256) >= (static_cast<int64_t>(1) << 31))
    return MOE_EUNSUPPORTED;
  moe::GemmArgs ga{};
  ga.part = reinterpret_cast<float*>(static_cast<char*>(ws) + l.part_off);
  ga.offsets = offsets;
  ga.a = dgu;
  ga.b0 = x;
  ga.row_token = row_token;
  ga.dw0 = dw_gate;
  ga.dw1 = dw_up;
  ga.accumulate = accumulate_dw;
  return from_hip(moe::launch_gemm(moe::GEMM_WGRAD_GATEUP, s, ga, stream));
}

moe_status moe_gemm_down_weighted(moe_shape s, const void* a, const int32_t* offsets, const void* w_down,
                                  const float* row_weight, void* o_perm, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(a, offsets, w_down, row_weight, o_perm)) return MOE_EINVAL;
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = a;
  ga.b0 = w_down;
  ga.row_weight = row_weight;
  ga.out0 = o_perm;
  return from_hip(moe::launch_gemm(moe::GEMM_DOWN, s, ga, stream));
}

moe_status moe_forward_fused(moe_shape s, const void* x, const void* w_router, const float* logit_bias,
                             const void* w_gate, const void* w_up, const void* w_down, float* logits,
                             int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                             int32_t* sorted_to_flat, int32_t* flat_to_sorted, int32_t* row_token, float* row_weight,
                             void* a, void* o_perm, void* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(x, w_router, w_gate, w_up, w_down, logits, topk_idx, topk_w, counts, offsets, sorted_to_flat,
               flat_to_sorted, row_token, row_weight, a, o_perm, y, ws))
    return MOE_EINVAL;
  if (!gathered_x_fits(s)) return MOE_EUNSUPPORTED;
  if (ws_bytes < moe::ws_layout(s).total) return MOE_EWORKSPACE;
  if ((st = moe_route(s, x, w_router, logit_bias, logits, topk_idx, topk_w, stream)) != MOE_OK) return st;
  if ((st = moe_permute_fused(s, topk_idx, topk_w, counts, offsets, sorted_to_flat, flat_to_sorted, row_token,
                              row_weight, ws, ws_bytes, stream)) != MOE_OK)
    return st;
  if ((st = moe_gemm_gate_up_gathered(s, x, row_token, offsets, w_gate, w_up, nullptr, nullptr, a, stream)) != MOE_OK)
    return st;
  if ((st = moe_gemm_down_weighted(s, a, offsets, w_down, row_weight, o_perm, stream)) != MOE_OK) return st;
  return moe_unpermute_sum(s, o_perm, flat_to_sorted, y, stream);
}

moe_status moe_forward_fused_noalloc(moe_shape s, const void* x, const void* w_router, const float* logit_bias,
                                     const void* w_gate, const void* w_up, const void* w_down, float* logits,
                                     int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                                     int32_t* sorted_to_flat, int32_t* flat_to_sorted, int32_t* row_token,
                                     float* row_weight, void* a, void* o_perm, void* y, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(x, w_router, w_gate, w_up, w_down, logits, topk_idx, topk_w, counts, offsets, sorted_to_flat,
               flat_to_sorted, row_token, row_weight, a, o_perm, y))
    return MOE_EINVAL;
  if (!gathered_x_fits(s)) return MOE_EUNSUPPORTED;
  if (moe::sort_hist_bytes(s) > moe::kScratchBytes) return MOE_EWORKSPACE;
  if ((st = moe_route(s, x, w_router, logit_bias, logits, topk_idx, topk_w, stream)) != MOE_OK) return st;
  if ((st = from_hip(moe::launch_permute_fused_noalloc(s, topk_idx, topk_w, counts, offsets, sorted_to_flat,
                                                       flat_to_sorted, row_token, row_weight, stream))) != MOE_OK)
    return st;
  if ((st = moe_gemm_gate_up_gathered(s, x, row_token, offsets, w_gate, w_up, nullptr, nullptr, a, stream)) != MOE_OK)
    return st;
  if ((st = moe_gemm_down_weighted(s, a, offsets, w_down, row_weight, o_perm, stream)) != MOE_OK) return st;
  return moe_unpermute_sum(s, o_perm, flat_to_sorted, y, stream);
}

moe_status moe_quantize_fp8_rows(int32_t rows, int32_t K, const void* in, uint8_t* q, uint8_t* e8,
                                 const int32_t* flat_to_sorted, int32_t k, hipStream_t stream) {
  if (rows < 0 || K <= 0 || K % 8 != 0) return MOE_EINVAL;
  if (any_null(in, q, e8)) return MOE_EINVAL;
  if (flat_to_sorted != nullptr && (k < 1 || static_cast<int64_t>(rows) * k >= (static_cast<int64_t>(1) << 31)))
    return MOE_EINVAL;
  return from_hip(moe::launch_quantize_fp8_rows(rows, K, in, q, e8, flat_to_sorted, k, stream));
}

namespace {
// The fp8 GEMMs: bf16 activations around them, K a multiple of their 64-wide
// k-step, the 8-bit x addressed with 32-bit byte offsets.
moe_status check_fp8_shape(const moe_shape& s) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s.dtype != MOE_BF16 || s.H % 64 != 0 || s.I % 64 != 0) return MOE_EUNSUPPORTED;
  if (static_cast<int64_t>(s.T) * s.H >= (static_cast<int64_t>(1) << 31)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}
}  // namespace

moe_status moe_gemm_gate_up_fp8(moe_shape s, const uint8_t* xq, const uint8_t* x_e8, const int32_t* row_token,
                                const int32_t* offsets, const uint8_t* wq_gate, const uint8_t* w_gate_e8,
                                const uint8_t* wq_up, const uint8_t* w_up_e8, void* a, hipStream_t stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(xq, x_e8, row_token, offsets, wq_gate, w_gate_e8, wq_up, w_up_e8, a)) return MOE_EINVAL;
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = xq;
  ga.a_scale = x_e8;
  ga.row_token = row_token;
  ga.b0 = wq_gate;
  ga.b0_scale = w_gate_e8;
  ga.b1 = wq_up;
  ga.b1_scale = w_up_e8;
  ga.out2 = a;
  return from_hip(moe::launch_gemm(moe::GEMM_GATEUP, s, ga, stream));
}

moe_status moe_gemm_down_fp8(moe_shape s, const uint8_t* aq, const uint8_t* a_e8, const int32_t* offsets,
                             const uint8_t* wq_down, const uint8_t* w_down_e8, const float* row_weight, void* o_perm,
                             hipStream_t stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(aq, a_e8, offsets, wq_down, w_down_e8, row_weight, o_perm)) return MOE_EINVAL;
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = aq;
  ga.a_scale = a_e8;
  ga.b0 = wq_down;
  ga.b0_scale = w_down_e8;
  ga.row_weight = row_weight;
  ga.out0 = o_perm;
  return from_hip(moe::launch_gemm(moe::GEMM_DOWN, s, ga, stream));
}

moe_status moe_forward_fused_fp8(moe_shape s, const void* x, const void* w_router, const float* logit_bias,
                                 const uint8_t* wq_gate, const uint8_t* w_gate_e8, const uint8_t* wq_up,
                                 const uint8_t* w_up_e8, const uint8_t* wq_down, const uint8_t* w_down_e8,
                                 float* logits, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                                 int32_t* sorted_to_flat, int32_t* flat_to_sorted, int32_t* row_token,
                                 float* row_weight, uint8_t* xq, uint8_t* x_e8, void* a, uint8_t* aq, uint8_t* a_e8,
                                 void* o_perm, void* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(x, w_router, wq_gate, w_gate_e8, wq_up, w_up_e8, wq_down, w_down_e8, logits, topk_idx, topk_w, counts,
               offsets, sorted_to_flat, flat_to_sorted, row_token, row_weight, xq, x_e8, a, aq, a_e8, o_perm, y, ws))
    return MOE_EINVAL;
  if (ws_bytes < moe::ws_layout(s).total) return MOE_EWORKSPACE;
  const int32_t M = s.T * s.k;
  if ((st = moe_route(s, x, w_router, logit_bias, logits, topk_idx, topk_w, stream)) != MOE_OK) return st;
  if ((st = moe_permute_fused(s, topk_idx, topk_w, counts, offsets, sorted_to_flat, flat_to_sorted, row_token,
                              row_weight, ws, ws_bytes, stream)) != MOE_OK)
    return st;
  if ((st = moe_quantize_fp8_rows(s.T, s.H, x, xq, x_e8, flat_to_sorted, s.k, stream)) != MOE_OK) return st;
  if ((st = moe_gemm_gate_up_fp8(s, xq, x_e8, row_token, offsets, wq_gate, w_gate_e8, wq_up, w_up_e8, a, stream)) !=
      MOE_OK)
    return st;
  if ((st = moe_quantize_fp8_rows(M, s.I, a, aq, a_e8, nullptr, 0, stream)) != MOE_OK) return st;
  if ((st = moe_gemm_down_fp8(s, aq, a_e8, offsets, wq_down, w_down_e8, row_weight, o_perm, stream)) != MOE_OK)
    return st;
  return moe_unpermute_sum(s, o_perm, flat_to_sorted, y, stream);
}

moe_status moe_gemm_gate_up_mxfp4(moe_shape s, const uint8_t* xq, const uint8_t* x_e8, const int32_t* row_token,
                                  const int32_t* offsets, const uint8_t* wq_gate, const uint8_t* w_gate_e8,
                                  const uint8_t* wq_up, const uint8_t* w_up_e8, void* a, hipStream_t stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(xq, x_e8, row_token, offsets, wq_gate, w_gate_e8, wq_up, w_up_e8, a)) return MOE_EINVAL;
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = xq;
  ga.a_scale = x_e8;
  ga.row_token = row_token;
  ga.b0 = wq_gate;
  ga.b0_scale = w_gate_e8;
  ga.b1 = wq_up;
  ga.b1_scale = w_up_e8;
  ga.b_fp4 = 1;
  ga.out2 = a;
  return from_hip(moe::launch_gemm(moe::GEMM_GATEUP, s, ga, stream));
}

moe_status moe_gemm_down_mxfp4(moe_shape s, const uint8_t* aq, const uint8_t* a_e8, const int32_t* offsets,
                               const uint8_t* wq_down, const uint8_t* w_down_e8, const float* row_weight,
                               void* o_perm, hipStream_t stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(aq, a_e8, offsets, wq_down, w_down_e8, row_weight, o_perm)) return MOE_EINVAL;
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = aq;
  ga.a_scale = a_e8;
  ga.b0 = wq_down;
  ga.b0_scale = w_down_e8;
  ga.b_fp4 = 1;
  ga.row_weight = row_weight;
  ga.out0 = o_perm;
  return from_hip(moe::launch_gemm(moe::GEMM_DOWN, s, ga, stream));
}

moe_status moe_forward_fused_mxfp4(moe_shape s, const void* x, const void* w_router, const float* logit_bias,
                                   const uint8_t* wq_gate, const uint8_t* w_gate_e8, const uint8_t* wq_up,
                                   const uint8_t* w_up_e8, const uint8_t* wq_down, const uint8_t* w_down_e8,
                                   float* logits, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                                   int32_t* sorted_to_flat, int32_t* flat_to_sorted, int32_t* row_token,
                                   float* row_weight, uint8_t* xq, uint8_t* x_e8, void* a, uint8_t* aq, uint8_t* a_e8,
                                   void* o_perm, void* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(x, w_router, wq_gate, w_gate_e8, wq_up, w_up_e8, wq_down, w_down_e8, logits, topk_idx, topk_w, counts,
               offsets, sorted_to_flat, flat_to_sorted, row_token, row_weight, xq, x_e8, a, aq, a_e8, o_perm, y, ws))
    return MOE_EINVAL;
  if (ws_bytes < moe::ws_layout(s).total) return MOE_EWORKSPACE;
  const int32_t M = s.T * s.k;
  if ((st = moe_route(s, x, w_router, logit_bias, logits, topk_idx, topk_w, stream)) != MOE_OK) return st;
  if ((st = moe_permute_fused(s, topk_idx, topk_w, counts, offsets, sorted_to_flat, flat_to_sorted, row_token,
                              row_weight, ws, ws_bytes, stream)) != MOE_OK)
    return st;
  if ((st = moe_quantize_fp8_rows(s.T, s.H, x, xq, x_e8, flat_to_sorted, s.k, stream)) != MOE_OK) return st;
  if ((st = moe_gemm_gate_up_mxfp4(s, xq, x_e8, row_token, offsets, wq_gate, w_gate_e8, wq_up, w_up_e8, a,
                                   stream)) != MOE_OK)
    return st;
  if ((st = moe_quantize_fp8_rows(M, s.I, a, aq, a_e8, nullptr, 0, stream)) != MOE_OK) return st;
  if ((st = moe_gemm_down_mxfp4(s, aq, a_e8, offsets, wq_down, w_down_e8, row_weight, o_perm, stream)) != MOE_OK)
    return st;
  return moe_unpermute_sum(s, o_perm, flat_to_sorted, y, stream);
}

moe_status moe_combine(moe_shape s, const void* o_perm, const float* topk_w, const int32_t* flat_to_sorted,
                       void* y, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(o_perm, topk_w, flat_to_sorted, y)) return MOE_EINVAL;
  return from_hip(moe::launch_combine(s, o_perm, topk_w, flat_to_sorted, y, stream));
}

moe_status moe_combine_bwd(moe_shape s, const void* dy, const void* o_perm, const float* topk_w,
                           const int32_t* flat_to_sorted, void* do_perm, float* d_topk_w, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(dy, o_perm, topk_w, flat_to_sorted, d_topk_w)) return MOE_EINVAL;  // do_perm may be NULL
  return from_hip(moe::launch_combine_bwd(s, dy, o_perm, topk_w, flat_to_sorted, do_perm, d_topk_w, stream));
}

moe_status moe_permute_rows(moe_shape s, const int32_t* topk_idx, const float* topk_w, const void* x,
                            int32_t* counts, int32_t* offsets, int32_t* sorted_to_flat, int32_t* flat_to_sorted,
                            int32_t* row_token, float* row_weight, void* x_perm, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(topk_idx, topk_w, x, counts, offsets, sorted_to_flat, flat_to_sorted, row_token, row_weight, x_perm,
               ws))
    return MOE_EINVAL;
  if (ws_bytes < moe::ws_layout(s).total) return MOE_EWORKSPACE;
  return from_hip(moe::launch_permute_rows(s, topk_idx, topk_w, x, counts, offsets, sorted_to_flat, flat_to_sorted,
                                           row_token, row_weight, x_perm, ws, stream));
}

moe_status moe_gemm_gate_up_aw(moe_shape s, const void* x_rows, const int32_t* row_token, const float* row_weight,
                               const int32_t* offsets, const void* w_gate, const void* w_up, void* g, void* u,
                               void* a, void* a_w, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(x_rows, row_weight, offsets, w_gate, w_up, g, u, a, a_w)) return MOE_EINVAL;
  if (s.dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (row_token != nullptr && !gathered_x_fits(s)) return MOE_EUNSUPPORTED;
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = x_rows;
  ga.row_token = row_token;
  ga.row_weight = row_weight;
  ga.b0 = w_gate;
  ga.b1 = w_up;
  ga.out0 = g;
  ga.out1 = u;
  ga.out2 = a;
  ga.out3 = a_w;
  return from_hip(moe::launch_gemm(moe::GEMM_GATEUP, s, ga, stream));
}

moe_status moe_gemm_down_bwd_dy(moe_shape s, const void* dy, const int32_t* row_token, const float* row_weight,
                                const void* a_w, const int32_t* offsets, const void* w_down, const void* g,
                                const void* u, void* dgu, float* dw_down, int accumulate_dw, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(dy, row_token, row_weight, a_w, offsets, w_down, g, u, dgu, dw_down, ws)) return MOE_EINVAL;
  if (accumulate_dw != 0 && accumulate_dw != 1) return MOE_EINVAL;
  if (s.dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  // dy rows are addressed with 32-bit byte offsets; the row tokens of the
  // weight gradient's k-rows are read up to two steps past the last row.
  if (!gathered_x_fits(s) || 4 * (static_cast<int64_t>(s.T) * s.k + 256) >= (static_cast<int64_t>(1) << 31))
    return MOE_EUNSUPPORTED;
  const WsLayout l = moe::ws_layout(s);
  if (ws_bytes < l.total) return MOE_EWORKSPACE;
  moe::GemmArgs gd{};
  gd.offsets = offsets;
  gd.a = dy;
  gd.row_token = row_token;
  gd.row_weight = row_weight;
  gd.b0 = w_down;
  gd.g_in = g;
  gd.u_in = u;
  gd.out0 = dgu;
  moe::GemmArgs gw{};
  gw.part = reinterpret_cast<float*>(static_cast<char*>(ws) + l.part_off);
  gw.offsets = offsets;
  gw.a = dy;
  gw.row_token = row_token;
  gw.b0 = a_w;
  gw.dw0 = dw_down;
  gw.accumulate = accumulate_dw;
  return from_hip(moe::launch_gemm_pair(moe::GEMM_DGRAD_DOWN, moe::GEMM_WGRAD_DOWN, s, gd, gw, stream));
}

moe_status moe_grouped_gemm_bwd(moe_shape s, const void* do_perm, const void* x_perm, const void* g, const void* u,
                                const void* a, const int32_t* offsets, const void* w_gate, const void* w_up,
                                const void* w_down, void* dx_perm, float* dw_gate, float* dw_up, float* dw_down,
                                int accumulate_dw, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(do_perm, x_perm, g, u, a, offsets, w_gate, w_up, w_down, dx_perm, dw_gate, dw_up, dw_down, ws))
    return MOE_EINVAL;
  if (accumulate_dw != 0 && accumulate_dw != 1) return MOE_EINVAL;
  const WsLayout l = moe::ws_layout(s);
  if (ws_bytes < l.total) return MOE_EWORKSPACE;
  void* dgu = static_cast<char*>(ws) + l.dgu_off;
  if ((st = moe_gemm_down_bwd(s, do_perm, a, offsets, w_down, g, u, dgu, dw_down, accumulate_dw, ws, ws_bytes,
                              stream)) != MOE_OK)
    return st;
  return moe_gemm_gate_up_bwd(s, dgu, x_perm, nullptr, offsets, w_gate, w_up, dx_perm, dw_gate, dw_up, accumulate_dw,
                              ws, ws_bytes, stream);
}

moe_status moe_gemm_down_bwd(moe_shape s, const void* do_perm, const void* a, const int32_t* offsets,
                             const void* w_down, const void* g, const void* u, void* dgu, float* dw_down,
                             int accumulate_dw, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(do_perm, a, offsets, w_down, g, u, dgu, dw_down, ws)) return MOE_EINVAL;
  if (accumulate_dw != 0 && accumulate_dw != 1) return MOE_EINVAL;
  const WsLayout l = moe::ws_layout(s);
  if (ws_bytes < l.total) return MOE_EWORKSPACE;
  moe::GemmArgs gd{};
  gd.offsets = offsets;
  gd.a = do_perm;
  gd.b0 = w_down;
  gd.g_in = g;
  gd.u_in = u;
  gd.out0 = dgu;
  moe::GemmArgs gw{};
  gw.part = reinterpret_cast<float*>(static_cast<char*>(ws) + l.part_off);
  gw.offsets = offsets;
  gw.a = do_perm;
  gw.b0 = a;
  gw.dw0 = dw_down;
  gw.accumulate = accumulate_dw;
  return from_hip(moe::launch_gemm_pair(moe::GEMM_DGRAD_DOWN, moe::GEMM_WGRAD_DOWN, s, gd, gw, stream));
}

moe_status moe_gemm_gate_up_bwd(moe_shape s, const void* dgu, const void* x_rows, const int32_t* row_token,
                                const int32_t* offsets, const void* w_gate, const void* w_up, void* dx_perm,
                                float* dw_gate, float* dw_up, int accumulate_dw, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(dgu, x_rows, offsets, w_gate, w_up, dx_perm, dw_gate, dw_up, ws)) return MOE_EINVAL;
  if (accumulate_dw != 0 && accumulate_dw != 1) return MOE_EINVAL;
  const WsLayout l = moe::ws_layout(s);
  if (ws_bytes < l.total) return MOE_EWORKSPACE;
  // Gathered x and row_token are addressed with 32-bit byte offsets.
  if (row_token != nullptr &&
      (static_cast<int64_t>(s.T) * s.H * (s.dtype == MOE_BF16 ? 2 : 4) >= (static_cast<int64_t>(1) << 31) ||
       4 * (static_cast<int64_t>(s.T) * s.k + 256) >= (static_cast<int64_t>(1) << 31)))
    return MOE_EUNSUPPORTED;
  moe::GemmArgs gd{};
  gd.offsets = offsets;
  gd.a = dgu;
  gd.b0 = w_gate;
  gd.b1 = w_up;
  gd.out0 = dx_perm;
  moe::GemmArgs gw{};
  gw.part = reinterpret_cast<float*>(static_cast<char*>(ws) + l.part_off);
  gw.offsets = offsets;
  gw.a = dgu;
  gw.b0 = x_rows;
  gw.row_token = row_token;
  gw.dw0 = dw_gate;
  gw.dw1 = dw_up;
  gw.accumulate = accumulate_dw;
  return from_hip(moe::launch_gemm_pair(moe::GEMM_DGRAD_GATEUP, moe::GEMM_WGRAD_GATEUP, s, gd, gw, stream));
}

moe_status moe_unpermute_sum(moe_shape s, const void* dx_perm, const int32_t* flat_to_sorted, void* dx,
                             hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(dx_perm, flat_to_sorted, dx)) return MOE_EINVAL;
  return from_hip(moe::launch_unpermute_sum(s, dx_perm, flat_to_sorted, dx, stream));
}

moe_status moe_route_bwd(moe_shape s, const float* d_topk_w, const float* topk_w, const int32_t* topk_idx,
                         float* d_logits, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(d_topk_w, topk_w, topk_idx, d_logits)) return MOE_EINVAL;
  return from_hip(moe::launch_route_bwd(s, d_topk_w, topk_w, topk_idx, d_logits, stream));
}

namespace {
// Adapter rank: a multiple of 8 (16-byte rows of B) up to 128 (the merge's
// LDS tile and the gradient kernels' register tiles).
moe_status check_lora(const moe_shape& s, int32_t r) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (r <= 0) return MOE_EINVAL;
  if (s.dtype != MOE_BF16 || r > 128 || r % 8 != 0) return MOE_EUNSUPPORTED;
  // The outer products address the sorted rows with 32-bit byte offsets.
  if (static_cast<int64_t>(s.T) * s.k * std::max(s.H, 2 * s.I) * 2 >= (static_cast<int64_t>(1) << 31))
    return MOE_EUNSUPPORTED;
  return MOE_OK;
}
}  // namespace

size_t moe_lora_workspace_bytes(moe_shape s, int32_t r) {
  if (check_lora(s, r) != MOE_OK) return 0;
  return moe::lora_layout(s, r).total;
}

moe_status moe_lora_merge(int32_t E, int32_t N, int32_t K, int32_t r, float scale, const void* w, const void* a,
                          const void* b, void* w_out, hipStream_t stream) {
  if (E <= 0 || N <= 0 || K <= 0 || r <= 0) return MOE_EINVAL;
  if (any_null(w, a, b, w_out)) return MOE_EINVAL;
  if (r > 128 || r % 8 != 0 || K % 8 != 0 || E > 65535 || (N + 127) / 128 > 65535) return MOE_EUNSUPPORTED;
  // One expert's weights are addressed with 32-bit byte offsets.
  // (Row tiles of a block reach up to 255 rows past the last; their loads
  // are range-checked and their results never stored.)
  if ((static_cast<int64_t>(N) + 256) * K >= (static_cast<int64_t>(1) << 30)) return MOE_EUNSUPPORTED;
  return from_hip(moe::launch_lora_merge(E, N, K, r, scale, w, a, b, w_out, stream));
}

moe_status moe_lora_merge_fp8(int32_t E, int32_t N, int32_t K, int32_t r, float scale, const uint8_t* wq,
                              const uint8_t* w_e8, const void* a, const void* b, void* w_out, hipStream_t stream) {
  if (E <= 0 || N <= 0 || K <= 0 || r <= 0) return MOE_EINVAL;
  if (any_null(wq, w_e8, a, b, w_out)) return MOE_EINVAL;
  if (r > 128 || r % 8 != 0 || K % 8 != 0 || E > 65535 || (N + 127) / 128 > 65535) return MOE_EUNSUPPORTED;
  if ((static_cast<int64_t>(N) + 256) * K >= (static_cast<int64_t>(1) << 30)) return MOE_EUNSUPPORTED;
  return from_hip(moe::launch_lora_merge_fp8(E, N, K, r, scale, wq, w_e8, a, b, w_out, stream));
}

moe_status moe_quantize_mxfp4_rows(int32_t rows, int32_t K, const void* in, uint8_t* q, uint8_t* e8,
                                   hipStream_t stream) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return MOE_EINVAL;
  if (any_null(in, q, e8)) return MOE_EINVAL;
  return from_hip(moe::launch_quantize_mxfp4_rows(rows, K, in, q, e8, 0, stream));
}

moe_status moe_quantize_mxfp4_weights(int32_t E, int32_t N, int32_t K, const void* w, uint8_t* q, uint8_t* e8,
                                      hipStream_t stream) {
  if (E <= 0 || N <= 0 || K <= 0 || K % 32 != 0) return MOE_EINVAL;
  if (any_null(w, q, e8)) return MOE_EINVAL;
  if (static_cast<int64_t>(E) * N >= (static_cast<int64_t>(1) << 31)) return MOE_EUNSUPPORTED;
  return from_hip(moe::launch_quantize_mxfp4_rows(E * N, K, w, q, e8, N, stream));
}

moe_status moe_lora_merge_mxfp4(int32_t E, int32_t N, int32_t K, int32_t r, float scale, const uint8_t* wq,
                                const uint8_t* w_e8, const void* a, const void* b, void* w_out, hipStream_t stream) {
  if (E <= 0 || N <= 0 || K <= 0 || r <= 0) return MOE_EINVAL;
  if (any_null(wq, w_e8, a, b, w_out)) return MOE_EINVAL;
  if (r > 128 || r % 8 != 0 || K % 32 != 0 || E > 65535 || (N + 127) / 128 > 65535) return MOE_EUNSUPPORTED;
  if ((static_cast<int64_t>(N) + 256) * K >= (static_cast<int64_t>(1) << 30)) return MOE_EUNSUPPORTED;
  return from_hip(moe::launch_lora_merge_mxfp4(E, N, K, r, scale, wq, w_e8, a, b, w_out, stream));
}

moe_status moe_lora_grads(moe_shape s, int32_t r, float scale, const void* x_perm, const void* act, const void* dgu,
                          const void* do_perm, const int32_t* offsets, const void* a_gate, const void* b_gate,
                          const void* a_up, const void* b_up, const void* a_down, const void* b_down, float* da_gate,
                          float* db_gate, float* da_up, float* db_up, float* da_down, float* db_down, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_lora(s, r);
  if (st != MOE_OK) return st;
  if (any_null(x_perm, act, dgu, do_perm, offsets, a_gate, b_gate, a_up, b_up, a_down, b_down, da_gate, db_gate,
               da_up, db_up, da_down, db_down, ws))
    return MOE_EINVAL;
  if (ws_bytes < moe::lora_layout(s, r).total) return MOE_EWORKSPACE;
  moe::LoraArgs g{};
  g.offsets = offsets;
  g.x_perm = x_perm;
  g.act = act;
  g.dgu = dgu;
  g.do_perm = do_perm;
  g.a_gate = a_gate;
  g.b_gate = b_gate;
  g.a_up = a_up;
  g.b_up = b_up;
  g.a_down = a_down;
  g.b_down = b_down;
  g.da_gate = da_gate;
  g.db_gate = db_gate;
  g.da_up = da_up;
  g.db_up = db_up;
  g.da_down = da_down;
  g.db_down = db_down;
  return from_hip(moe::launch_lora_grads(s, r, scale, g, ws, stream));
}

// ---- The adapter step without merged weights --------------------------------
namespace {
// check_lora, the K extensions' rows [T*k][2rp] addressed with 32-bit byte
// offsets, and the workspace.
moe_status check_lora_unmerged(const moe_shape& s, int32_t r, size_t ws_bytes) {
  const moe_status st = check_lora(s, r);
  if (st != MOE_OK) return st;
  if (static_cast<int64_t>(s.T) * s.k * 4 * moe::lora_padded_rank(r) >= (static_cast<int64_t>(1) << 31))
    return MOE_EUNSUPPORTED;
  if (ws_bytes < moe::lora_layout(s, r).total) return MOE_EWORKSPACE;
  return MOE_OK;
}
void* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }
}  // namespace

size_t moe_lora_unmerged_workspace_bytes(moe_shape s, int32_t r) {
  if (check_lora_unmerged(s, r, ~static_cast<size_t>(0)) != MOE_OK) return 0;
  return moe::lora_layout(s, r).total;
}

moe_status moe_lora_prepare(moe_shape s, int32_t r, float scale, const void* a_gate, const void* b_gate,
                            const void* a_up, const void* b_up, const void* a_down, const void* b_down, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  const moe_status st = check_lora_unmerged(s, r, ws_bytes);
  if (st != MOE_OK) return st;
  if (any_null(a_gate, b_gate, a_up, b_up, a_down, b_down, ws)) return MOE_EINVAL;
  moe::LoraArgs g{};
  g.a_gate = a_gate;
  g.b_gate = b_gate;
  g.a_up = a_up;
  g.b_up = b_up;
  g.a_down = a_down;
  g.b_down = b_down;
  return from_hip(moe::launch_lora_prepare(s, r, scale, g, ws, stream));
}

moe_status moe_lora_gemm_gate_up(moe_shape s, int32_t r, const void* x_perm, const int32_t* offsets,
                                 const void* w_gate, const void* w_up, const void* b_gate, const void* b_up, void* g,
                                 void* u, void* a, void* ws, size_t ws_bytes, hipStream_t stream) {
  const moe_status st = check_lora_unmerged(s, r, ws_bytes);
  if (st != MOE_OK) return st;
  if (any_null(x_perm, offsets, w_gate, w_up, b_gate, b_up, g, u, a, ws)) return MOE_EINVAL;
  const moe::LoraLayout l = moe::lora_layout(s, r);
  hipError_t err = moe::launch_lora_project(s, r, 0, x_perm, offsets, ws, stream);  // Z_gu
  if (err != hipSuccess) return from_hip(err);
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = x_perm;
  ga.b0 = w_gate;
  ga.b1 = w_up;
  ga.out0 = g;
  ga.out1 = u;
  ga.out2 = a;
  ga.ax = at(ws, l.z_gu);
  ga.bx0 = b_gate;
  ga.bx1 = b_up;
  ga.kxr = r;
  ga.kxp = moe::lora_padded_rank(r);
  ga.kx = 2 * ga.kxp;
  return from_hip(moe::launch_gemm(moe::GEMM_GATEUP, s, ga, stream));
}

moe_status moe_lora_gemm_down(moe_shape s, int32_t r, const void* a, const int32_t* offsets, const void* w_down,
                              const void* b_down, void* o_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  const moe_status st = check_lora_unmerged(s, r, ws_bytes);
  if (st != MOE_OK) return st;
  if (any_null(a, offsets, w_down, b_down, o_perm, ws)) return MOE_EINVAL;
  const moe::LoraLayout l = moe::lora_layout(s, r);
  hipError_t err = moe::launch_lora_project(s, r, 2, a, offsets, ws, stream);  // Z_d
  if (err != hipSuccess) return from_hip(err);
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = a;
  ga.b0 = w_down;
  ga.out0 = o_perm;
  ga.ax = at(ws, l.z_d);
  ga.bx0 = b_down;
  ga.kxr = r;
  ga.kxp = ga.kx = moe::lora_padded_rank(r);
  return from_hip(moe::launch_gemm(moe::GEMM_DOWN, s, ga, stream));
}

moe_status moe_lora_gemm_down_dgrad(moe_shape s, int32_t r, const void* do_perm, const int32_t* offsets,
                                    const void* w_down, const void* a_down, const void* g, const void* u, void* dgu,
                                    void* ws, size_t ws_bytes, hipStream_t stream) {
  const moe_status st = check_lora_unmerged(s, r, ws_bytes);
  if (st != MOE_OK) return st;
  if (any_null(do_perm, offsets, w_down, a_down, g, u, dgu, ws)) return MOE_EINVAL;
  const moe::LoraLayout l = moe::lora_layout(s, r);
  hipError_t err = moe::launch_lora_project(s, r, 3, do_perm, offsets, ws, stream);  // Y_d
  if (err != hipSuccess) return from_hip(err);
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = do_perm;
  ga.b0 = w_down;
  ga.g_in = g;
  ga.u_in = u;
  ga.out0 = dgu;
  ga.ax = at(ws, l.y_d);
  ga.bx0 = a_down;
  ga.kxr = r;
  ga.kxp = ga.kx = moe::lora_padded_rank(r);
  return from_hip(moe::launch_gemm(moe::GEMM_DGRAD_DOWN, s, ga, stream));
}

moe_status moe_lora_gemm_gate_up_dgrad(moe_shape s, int32_t r, const void* dgu, const int32_t* offsets,
                                       const void* w_gate, const void* w_up, const void* a_gate, const void* a_up,
                                       void* dx_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  const moe_status st = check_lora_unmerged(s, r, ws_bytes);
  if (st != MOE_OK) return st;
  if (any_null(dgu, offsets, w_gate, w_up, a_gate, a_up, dx_perm, ws)) return MOE_EINVAL;
  const moe::LoraLayout l = moe::lora_layout(s, r);
  hipError_t err = moe::launch_lora_project(s, r, 1, dgu, offsets, ws, stream);  // Y_gu
  if (err != hipSuccess) return from_hip(err);
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = dgu;
  ga.b0 = w_gate;
  ga.b1 = w_up;
  ga.out0 = dx_perm;
  ga.ax = at(ws, l.y_gu);
  ga.bx0 = a_gate;
  ga.bx1 = a_up;
  ga.kxr = r;
  ga.kxp = moe::lora_padded_rank(r);
  ga.kx = 2 * ga.kxp;
  return from_hip(moe::launch_gemm(moe::GEMM_DGRAD_GATEUP, s, ga, stream));
}

moe_status moe_lora_gemm_gate_up_gathered(moe_shape s, int32_t r, const void* x, const int32_t* row_token,
                                          const int32_t* offsets, const void* w_gate, const void* w_up,
                                          const void* b_gate, const void* b_up, void* g, void* u, void* a, void* ws,
                                          size_t ws_bytes, hipStream_t stream) {
  const moe_status st = check_lora_unmerged(s, r, ws_bytes);
  if (st != MOE_OK) return st;
  if (any_null(x, row_token, offsets, w_gate, w_up, b_gate, b_up, g, u, a, ws)) return MOE_EINVAL;
  // x's rows (and dy's, in the calls below) are addressed with 32-bit byte
  // offsets: check_lora's bound on the sorted rows (T k >= T of them) covers them.
  const moe::LoraLayout l = moe::lora_layout(s, r);
  hipError_t err = moe::launch_lora_project(s, r, 0, x, offsets, ws, stream, row_token);  // Z_gu from x's rows
  if (err != hipSuccess) return from_hip(err);
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = x;
  ga.row_token = row_token;
  ga.b0 = w_gate;
  ga.b1 = w_up;
  ga.out0 = g;
  ga.out1 = u;
  ga.out2 = a;
  ga.ax = at(ws, l.z_gu);
  ga.bx0 = b_gate;
  ga.bx1 = b_up;
  ga.kxr = r;
  ga.kxp = moe::lora_padded_rank(r);
  ga.kx = 2 * ga.kxp;
  return from_hip(moe::launch_gemm(moe::GEMM_GATEUP, s, ga, stream));
}

moe_status moe_lora_gemm_down_dgrad_dy(moe_shape s, int32_t r, const void* dy, const int32_t* row_token,
                                       const float* row_weight, const int32_t* offsets, const void* w_down,
                                       const void* a_down, const void* g, const void* u, void* dgu, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
  const moe_status st = check_lora_unmerged(s, r, ws_bytes);
  if (st != MOE_OK) return st;
  if (any_null(dy, row_token, row_weight, offsets, w_down, a_down, g, u, dgu, ws)) return MOE_EINVAL;
  const moe::LoraLayout l = moe::lora_layout(s, r);
  // dy's rows through the tokens, unweighted: the kernel applies the
  // routing weight to the whole sum, extension included.
  hipError_t err = moe::launch_lora_project(s, r, 3, dy, offsets, ws, stream, row_token);
  if (err != hipSuccess) return from_hip(err);
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = dy;
  ga.row_token = row_token;
  ga.row_weight = row_weight;
  ga.b0 = w_down;
  ga.g_in = g;
  ga.u_in = u;
  ga.out0 = dgu;
  ga.ax = at(ws, l.y_d);
  ga.bx0 = a_down;
  ga.kxr = r;
  ga.kxp = ga.kx = moe::lora_padded_rank(r);
  return from_hip(moe::launch_gemm(moe::GEMM_DGRAD_DOWN, s, ga, stream));
}

moe_status moe_lora_grads_unmerged_gathered(moe_shape s, int32_t r, const void* x, const int32_t* row_token,
                                            const float* row_weight, const void* act, const void* dgu, const void* dy,
                                            const int32_t* offsets, float* da_gate, float* db_gate, float* da_up,
                                            float* db_up, float* da_down, float* db_down, void* ws, size_t ws_bytes,
                                            hipStream_t stream) {
  const moe_status st = check_lora_unmerged(s, r, ws_bytes);
  if (st != MOE_OK) return st;
  if (any_null(x, row_token, row_weight, act, dgu, dy, offsets, da_gate, db_gate, da_up, db_up, da_down, db_down, ws))
    return MOE_EINVAL;
  // The two projections that carry dO = w dy, again with the weight: Z_down'
  // = w Z_down (for dB_down = dy^T Z_down') and Y_down = w (dy sB_down).
  hipError_t err = moe::launch_lora_project(s, r, 2, act, offsets, ws, stream, nullptr, row_weight);
  if (err == hipSuccess) err = moe::launch_lora_project(s, r, 3, dy, offsets, ws, stream, row_token, row_weight);
  if (err != hipSuccess) return from_hip(err);
  moe::LoraArgs g{};
  g.offsets = offsets;
  g.x_perm = x;
  g.act = act;
  g.dgu = dgu;
  g.do_perm = dy;
  g.row_token = row_token;
  g.row_weight = row_weight;
  g.da_gate = da_gate;
  g.db_gate = db_gate;
  g.da_up = da_up;
  g.db_up = db_up;
  g.da_down = da_down;
  g.db_down = db_down;
  return from_hip(moe::launch_lora_outer(s, r, g, ws, stream));
}

moe_status moe_lora_grads_unmerged(moe_shape s, int32_t r, const void* x_perm, const void* act, const void* dgu,
                                   const void* do_perm, const int32_t* offsets, float* da_gate, float* db_gate,
                                   float* da_up, float* db_up, float* da_down, float* db_down, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  const moe_status st = check_lora_unmerged(s, r, ws_bytes);
  if (st != MOE_OK) return st;
  if (any_null(x_perm, act, dgu, do_perm, offsets, da_gate, db_gate, da_up, db_up, da_down, db_down, ws))
    return MOE_EINVAL;
  moe::LoraArgs g{};
  g.offsets = offsets;
  g.x_perm = x_perm;
  g.act = act;
  g.dgu = dgu;
  g.do_perm = do_perm;
  g.da_gate = da_gate;
  g.db_gate = db_gate;
  g.da_up = da_up;
  g.db_up = db_up;
  g.da_down = da_down;
  g.db_down = db_down;
  return from_hip(moe::launch_lora_outer(s, r, g, ws, stream));
}

moe_status moe_lora_grads_gathered(moe_shape s, int32_t r, float scale, const void* x, const int32_t* row_token,
                                   const float* row_weight, const void* act, const void* dgu, const void* dy,
                                   const int32_t* offsets, const void* a_gate, const void* b_gate, const void* a_up,
                                   const void* b_up, const void* a_down, const void* b_down, float* da_gate,
                                   float* db_gate, float* da_up, float* db_up, float* da_down, float* db_down,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_lora(s, r);
  if (st != MOE_OK) return st;
  if (any_null(x, row_token, row_weight, act, dgu, dy, offsets, a_gate, b_gate, a_up, b_up, a_down, b_down, da_gate,
               db_gate, da_up, db_up, da_down, db_down, ws))
    return MOE_EINVAL;
  if (ws_bytes < moe::lora_layout(s, r).total) return MOE_EWORKSPACE;
  moe::LoraArgs g{};
  g.offsets = offsets;
  g.x_perm = x;
  g.act = act;
  g.dgu = dgu;
  g.do_perm = dy;
  g.row_token = row_token;
  g.row_weight = row_weight;
  g.a_gate = a_gate;
  g.b_gate = b_gate;
  g.a_up = a_up;
  g.b_up = b_up;
  g.a_down = a_down;
  g.b_down = b_down;
  g.da_gate = da_gate;
  g.db_gate = db_gate;
  g.da_up = da_up;
  g.db_up = db_up;
  g.da_down = da_down;
  g.db_down = db_down;
  return from_hip(moe::launch_lora_grads(s, r, scale, g, ws, stream));
}

moe_status moe_gemm_down_dgrad_dy(moe_shape s, const void* dy, const int32_t* row_token, const float* row_weight,
                                  const int32_t* offsets, const void* w_down, const void* g, const void* u, void* dgu,
                                  hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (any_null(dy, row_token, row_weight, offsets, w_down, g, u, dgu)) return MOE_EINVAL;
  if (s.dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (!gathered_x_fits(s)) return MOE_EUNSUPPORTED;  // dy rows: 32-bit byte offsets
  moe::GemmArgs ga{};
  ga.offsets = offsets;
  ga.a = dy;
  ga.row_token = row_token;
  ga.row_weight = row_weight;
  ga.b0 = w_down;
  ga.g_in = g;
  ga.u_in = u;
  ga.out0 = dgu;
  return from_hip(moe::launch_gemm(moe::GEMM_DGRAD_DOWN, s, ga, stream));
}

}  // extern "C"
