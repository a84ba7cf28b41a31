// Expert GEMMs for the float32 dtype: one thread per output element on the
// vector ALUs, fp32 accumulation in ascending k. This dtype serves small
// problems (the tiny fp32 layer); the bf16 dtype runs on the matrix cores
// (gemm_bf16.hip). Both compute the same per-expert products over the rows
// that moe_permute sorted by expert.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// The expert whose row range [offsets[e], offsets[e+1]) holds row p: the last
// e with offsets[e] <= p (empty experts share their offset with the next).
__device__ __forceinline__ int expert_of_row(int p, const int32_t* __restrict__ offsets, int E) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// row_token (fused forward): row p of the input is row row_token[p] of x;
// g and u may then be null (A only).
__global__ __launch_bounds__(kThreads) void gateup_f32(int rows, int H, int E, int I, const int32_t* offsets,
                                                       const float* __restrict__ xp,
                                                       const int32_t* __restrict__ row_token,
                                                       const float* __restrict__ wg, const float* __restrict__ wu,
                                                       float* __restrict__ g, float* __restrict__ u,
                                                       float* __restrict__ a) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (q >= static_cast<int64_t>(rows) * I) return;
  const int p = static_cast<int>(q / I), i = static_cast<int>(q % I);
  const int e = expert_of_row(p, offsets, E);
  const float* x = xp + static_cast<int64_t>(row_token ? row_token[p] : p) * H;
  const float* rg = wg + (static_cast<int64_t>(e) * I + i) * H;
  const float* ru = wu + (static_cast<int64_t>(e) * I + i) * H;
  float sg = 0.0f, su = 0.0f;
  for (int h = 0; h < H; ++h) {
    sg += x[h] * rg[h];
    su += x[h] * ru[h];
  }
  if (g) g[q] = sg;
  if (u) u[q] = su;
  a[q] = sg * sigmoidf_dev(sg) * su;
}

// row_weight (fused forward): output row p scaled by row_weight[p].
__global__ __launch_bounds__(kThreads) void down_f32(int rows, int H, int E, int I, const int32_t* offsets,
                                                     const float* __restrict__ act, const float* __restrict__ wd,
                                                     const float* __restrict__ row_weight, float* __restrict__ o) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (q >= static_cast<int64_t>(rows) * H) return;
  const int p = static_cast<int>(q / H), h = static_cast<int>(q % H);
  const int e = expert_of_row(p, offsets, E);
  const float* av = act + static_cast<int64_t>(p) * I;
  const float* r = wd + (static_cast<int64_t>(e) * H + h) * I;
  float s = 0.0f;
  for (int i = 0; i < I; ++i) s += av[i] * r[i];
  o[q] = row_weight ? s * row_weight[p] : s;
}

// dA = dO W_down[e]; dU = dA silu(g); dG = dA u s (1 + g (1 - s)) -> dgu = [dG | dU]
__global__ __launch_bounds__(kThreads) void dgrad_down_f32(int rows, int H, int E, int I, const int32_t* offsets,
                                                           const float* __restrict__ dop,
                                                           const float* __restrict__ wd,
                                                           const float* __restrict__ g,
                                                           const float* __restrict__ u, float* __restrict__ dgu) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (q >= static_cast<int64_t>(rows) * I) return;
  const int p = static_cast<int>(q / I), i = static_cast<int>(q % I);
  const int e = expert_of_row(p, offsets, E);
  const float* d = dop + static_cast<int64_t>(p) * H;
  const float* w = wd + static_cast<int64_t>(e) * H * I + i;
  float da = 0.0f;
  for (int h = 0; h < H; ++h) da += d[h] * w[static_cast<int64_t>(h) * I];
  const float gv = g[q], uv = u[q];
  const float s = sigmoidf_dev(gv);
  dgu[static_cast<int64_t>(p) * 2 * I + i] = da * uv * s * (1.0f + gv * (1.0f - s));
  dgu[static_cast<int64_t>(p) * 2 * I + I + i] = da * (gv * s);
}

// dx_perm = dG W_gate[e] + dU W_up[e]
__global__ __launch_bounds__(kThreads) void dgrad_gateup_f32(int rows, int H, int E, int I, const int32_t* offsets,
                                                             const float* __restrict__ dgu,
                                                             const float* __restrict__ wg,
                                                             const float* __restrict__ wu,
                                                             float* __restrict__ dxp) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (q >= static_cast<int64_t>(rows) * H) return;
  const int p = static_cast<int>(q / H), h = static_cast<int>(q % H);
  const int e = expert_of_row(p, offsets, E);
  const float* d = dgu + static_cast<int64_t>(p) * 2 * I;
  const float* g = wg + static_cast<int64_t>(e) * I * H + h;
  const float* u = wu + static_cast<int64_t>(e) * I * H + h;
  float s = 0.0f;
  for (int i = 0; i < I; ++i) s += d[i] * g[static_cast<int64_t>(i) * H];
  for (int i = 0; i < I; ++i) s += d[I + i] * u[static_cast<int64_t>(i) * H];
  dxp[q] = s;
}

// dW_down[e][h][i] = sum_p dO[p][h] act[p][i]
__global__ __launch_bounds__(kThreads) void wgrad_down_f32(int H, int E, int I, const int32_t* offsets,
                                                           const float* __restrict__ dop,
                                                           const float* __restrict__ act, float* __restrict__ dw,
                                                           int accumulate) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t per = static_cast<int64_t>(H) * I;
  if (q >= per * E) return;
  const int e = static_cast<int>(q / per);
  const int h = static_cast<int>((q % per) / I), i = static_cast<int>(q % I);
  float s = 0.0f;
  for (int p = offsets[e]; p < offsets[e + 1]; ++p)
    s += dop[static_cast<int64_t>(p) * H + h] * act[static_cast<int64_t>(p) * I + i];
  dw[q] = accumulate ? dw[q] + s : s;
}

// dW_gate[e][i][h] = sum_p dG[p][i] x[p][h]; dW_up likewise with dU. With
// row_token, row p of x is row row_token[p] of the unsorted x.
__global__ __launch_bounds__(kThreads) void wgrad_gateup_f32(int H, int E, int I, const int32_t* offsets,
                                                             const float* __restrict__ dgu,
                                                             const float* __restrict__ xp,
                                                             const int32_t* __restrict__ row_token,
                                                             float* __restrict__ dwg, float* __restrict__ dwu,
                                                             int accumulate) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t per = 2ll * I * H;
  if (q >= per * E) return;
  const int e = static_cast<int>(q / per);
  const int m = static_cast<int>((q % per) / H), h = static_cast<int>(q % H);
  float s = 0.0f;
  for (int p = offsets[e]; p < offsets[e + 1]; ++p)
    s += dgu[static_cast<int64_t>(p) * 2 * I + m] * xp[static_cast<int64_t>(row_token ? row_token[p] : p) * H + h];
  float* out = (m < I) ? dwg + (static_cast<int64_t>(e) * I + m) * H + h
                       : dwu + (static_cast<int64_t>(e) * I + (m - I)) * H + h;
  *out = accumulate ? *out + s : s;
}

inline unsigned blocks_for(int64_t n) { return static_cast<unsigned>(ceil_div64(n, kThreads)); }

}  // namespace

hipError_t launch_gemm_f32(GemmMode mode, const moe_shape& s, const GemmArgs& g, hipStream_t st) {
  const int rows = s.T * s.k;
  const float* A = static_cast<const float*>(g.a);
  const float* B0 = static_cast<const float*>(g.b0);
  const float* B1 = static_cast<const float*>(g.b1);
  switch (mode) {
    case GEMM_GATEUP:
      gateup_f32<<<blocks_for(static_cast<int64_t>(rows) * s.I), kThreads, 0, st>>>(
          rows, s.H, s.E, s.I, g.offsets, A, g.row_token, B0, B1, static_cast<float*>(g.out0),
          static_cast<float*>(g.out1), static_cast<float*>(g.out2));
      break;
    case GEMM_DOWN:
      down_f32<<<blocks_for(static_cast<int64_t>(rows) * s.H), kThreads, 0, st>>>(
          rows, s.H, s.E, s.I, g.offsets, A, B0, g.row_weight, static_cast<float*>(g.out0));
      break;
    case GEMM_DGRAD_DOWN:
      dgrad_down_f32<<<blocks_for(static_cast<int64_t>(rows) * s.I), kThreads, 0, st>>>(
          rows, s.H, s.E, s.I, g.offsets, A, B0, static_cast<const float*>(g.g_in),
          static_cast<const float*>(g.u_in), static_cast<float*>(g.out0));
      break;
    case GEMM_DGRAD_GATEUP:
      dgrad_gateup_f32<<<blocks_for(static_cast<int64_t>(rows) * s.H), kThreads, 0, st>>>(
          rows, s.H, s.E, s.I, g.offsets, A, B0, B1, static_cast<float*>(g.out0));
      break;
    case GEMM_WGRAD_DOWN:
      wgrad_down_f32<<<blocks_for(static_cast<int64_t>(s.E) * s.H * s.I), kThreads, 0, st>>>(
          s.H, s.E, s.I, g.offsets, A, B0, g.dw0, g.accumulate);
      break;
    case GEMM_WGRAD_GATEUP:
      wgrad_gateup_f32<<<blocks_for(2ll * s.E * s.I * s.H), kThreads, 0, st>>>(
          s.H, s.E, s.I, g.offsets, A, B0, g.row_token, g.dw0, g.dw1, g.accumulate);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
