// CPU oracle for one MoE layer's expert stage, forward and backward.
//
// TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
// benchmark's CPU-baseline leg may load this library. The product path (the
// HIP library) never calls it, and the two share no code: no headers, no
// helpers, no tables.
//
// What it computes is the plain definition of the stage, with no blocking,
// fusion or reordering:
//   * router (torchtune PR #2820 "[WIP] Qwen3 MoE support", comment on the
//     top-score renormalisation; axolotl issue #3155, comments on the router
//     weight shape [E, H] = nn.Linear(H, E); sourcepulse summary, "Highlighted
//     Details": fused softmax + top-k): logits = x . Wr^T (+ bias), softmax
//     over the E experts, the k largest kept and renormalised by their sum
//     plus 1e-20;
//   * expert indexing (unsloth PR #3812, review suggestion that replaces the
//     one-hot counting with a stable argsort of the flattened expert ids and a
//     bincount): counts, offsets, and the stable permutation of the T*k
//     (token, slot) pairs by expert;
//   * experts (unsloth PR #3812, the stacked weights gate_up [E, 2I, H] and
//     down [E, H, I], held here as separate W_gate, W_up [E, I, H] and W_down
//     [E, H, I]; axolotl issue #3155, numerical-check comment: no bias, silu
//     gating): A = silu(X W_gate^T) * (X W_up^T), O = A W_down^T;
//   * combine (modelopt.torch.utils.moe, a2a_moe: each token's k expert
//     results are weighted by its routing weights, kept in the weights' own
//     precision, and summed): Y[t] = sum_j w[t,j] O[t,j];
//   * the backward of all of the above by the chain rule.
//
// Arithmetic: every reduction is a sequential loop in ascending index order.
// GEMMs run in axpy order (for each output row: for each k: row += a[k] *
// b[k, :]), so each output element is a sequential sum over k; running the
// inner loop over independent output elements (which the compiler may
// vectorise) does not reorder any sum. Build with -ffp-contract=off and
// without fast-math so every mul and add is rounded as written. std::thread
// splits independent outputs (tokens, expert rows) across cores, which changes
// no arithmetic order.
//
// The router logit is the one value that must match the HIP path bit for bit;
// it is defined as acc = +0; for h ascending: acc = fma(x[t,h], Wr[e,h], acc);
// then acc + bias[e]. With bf16 inputs each product is exact in fp32, so the
// fma equals a multiply-add; for fp32 inputs the fma is part of the
// definition.
//
// Parity pins (the test suite, not this file): brute force on tiny inputs
// (every expert run densely on every token, then masked), library autograd
// in float64, central finite differences in float64, closed-form invariants
// (weights sum to 1, counts sum to T*k, permutations are mutual inverses,
// gather followed by combine is the identity), and special cases E = k = 1
// (a dense SwiGLU MLP) and k = E (the full softmax).

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

namespace {

int g_threads = 0;  // 0: use every hardware thread

int thread_count() {
  if (g_threads > 0) return g_threads;
  unsigned n = std::thread::hardware_concurrency();
  return n == 0 ? 1 : static_cast<int>(n);
}

// Runs fn(i) for i in [0, n) on a pool of threads; each i is independent.
void parallel_for(int64_t n, const std::function<void(int64_t)>& fn) {
  int nt = thread_count();
  if (nt <= 1 || n <= 1) {
    for (int64_t i = 0; i < n; ++i) fn(i);
    return;
  }
  if (nt > n) nt = static_cast<int>(n);
  std::atomic<int64_t> next(0);
  std::vector<std::thread> pool;
  pool.reserve(nt);
  for (int w = 0; w < nt; ++w) {
    pool.emplace_back([&]() {
      for (;;) {
        int64_t i = next.fetch_add(1);
        if (i >= n) break;
        fn(i);
      }
    });
  }
  for (auto& th : pool) th.join();
}

template <class R> R fused_mul_add(R a, R b, R c);
template <> float fused_mul_add<float>(float a, float b, float c) { return std::fmaf(a, b, c); }
template <> double fused_mul_add<double>(double a, double b, double c) { return std::fma(a, b, c); }

template <class R> R expo(R v);
template <> float expo<float>(float v) { return std::exp(v); }
template <> double expo<double>(double v) { return std::exp(v); }

template <class R> R sigmoid(R g) { return R(1) / (R(1) + expo<R>(-g)); }

// ----------------------------------------------------------------------------
// Router: logits, top-k selection, softmax, renormalised top-k weights.
// ----------------------------------------------------------------------------
template <class R>
int route(int T, int H, int E, int k, const R* x, const R* wr, const R* bias,
          R* logits, int32_t* idx, R* w) {
  if (T < 0 || H <= 0 || E <= 0 || k <= 0 || k > E) return 1;
  parallel_for(T, [&](int64_t t) {
    R* l = logits + t * E;
    const R* xt = x + t * H;
    for (int e = 0; e < E; ++e) {
      const R* we = wr + static_cast<int64_t>(e) * H;
      R acc = R(0);
      for (int h = 0; h < H; ++h) acc = fused_mul_add<R>(xt[h], we[h], acc);
      if (bias) acc = acc + bias[e];
      l[e] = acc;
    }
    // Selection on the logits (softmax is monotone in them): the largest
    // first; among equal logits the lower expert index first. A NaN logit
    // ranks below every number, -inf included (among NaNs, the lower index).
    auto above = [](R a, R b) {
      if (std::isnan(b)) return !std::isnan(a);
      return !std::isnan(a) && a > b;
    };
    std::vector<char> taken(E, 0);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || above(l[e], l[best])) best = e;
      }
      taken[best] = 1;
      idx[t * k + j] = best;
    }
    // Softmax over all E logits, shifted by their maximum.
    R m = l[0];
    for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
    R z = R(0);
    for (int e = 0; e < E; ++e) z = z + expo<R>(l[e] - m);
    // Renormalise the kept probabilities by their sum plus 1e-20.
    std::vector<R> p(k);
    R s = R(0);
    for (int j = 0; j < k; ++j) {
      p[j] = expo<R>(l[idx[t * k + j]] - m) / z;
      s = s + p[j];
    }
    R den = s + R(1e-20);
    for (int j = 0; j < k; ++j) w[t * k + j] = p[j] / den;
  });
  return 0;
}

// ----------------------------------------------------------------------------
// Expert indexing: counts, offsets and the stable permutation by expert.
// pos(f) = offsets[e_f] + #{f' < f : e_f' == e_f}.
// ----------------------------------------------------------------------------
int permute_index(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                  int32_t* sorted_to_flat, int32_t* flat_to_sorted) {
  if (T < 0 || E <= 0 || k <= 0) return 1;
  const int64_t n = static_cast<int64_t>(T) * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < n; ++f) {
    int32_t e = idx[f];
    if (e < 0 || e >= E) return 2;
    counts[e] += 1;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> fill(offsets, offsets + E);
  for (int64_t f = 0; f < n; ++f) {
    int32_t p = fill[idx[f]]++;
    sorted_to_flat[p] = static_cast<int32_t>(f);
    flat_to_sorted[f] = p;
  }
  return 0;
}

// X_perm[p, :] = X[sorted_to_flat[p] / k, :]
template <class R>
void gather_rows(int T, int H, int k, const R* x, const int32_t* sorted_to_flat, R* x_perm) {
  const int64_t n = static_cast<int64_t>(T) * k;
  parallel_for(n, [&](int64_t p) {
    const R* src = x + static_cast<int64_t>(sorted_to_flat[p] / k) * H;
    std::memcpy(x_perm + p * H, src, sizeof(R) * H);
  });
}

// Transposes one [rows, cols] matrix into [cols, rows].
template <class R>
std::vector<R> transposed(const R* a, int rows, int cols) {
  std::vector<R> t(static_cast<size_t>(rows) * cols);
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) t[static_cast<size_t>(c) * rows + r] = a[static_cast<size_t>(r) * cols + c];
  return t;
}

// out[0:n] = sum over kk ascending of a[kk] * b[kk*n : kk*n + n]   (axpy order)
template <class R>
void row_times_matrix(const R* a, int64_t K, const R* b, int64_t n, R* out) {
  for (int64_t j = 0; j < n; ++j) out[j] = R(0);
  for (int64_t kk = 0; kk < K; ++kk) {
    const R av = a[kk];
    const R* br = b + kk * n;
    for (int64_t j = 0; j < n; ++j) out[j] = out[j] + av * br[j];
  }
}

// ----------------------------------------------------------------------------
// Experts forward over the sorted rows: for each expert e and row p in
// [offsets[e], offsets[e+1]): G = X_perm W_gate[e]^T, U = X_perm W_up[e]^T,
// A = G * sigmoid(G) * U, O = A W_down[e]^T.  expert_mask (optional, [E])
// restricts the work to the marked experts; other rows are left untouched.
// ----------------------------------------------------------------------------
template <class R>
void experts_fwd(int H, int E, int I, const R* x_perm, const int32_t* offsets, const R* w_gate,
                 const R* w_up, const R* w_down, const uint8_t* expert_mask, R* g, R* u, R* a, R* o) {
  for (int e = 0; e < E; ++e) {
    if (expert_mask && !expert_mask[e]) continue;
    const int64_t r0 = offsets[e], r1 = offsets[e + 1];
    if (r1 <= r0) continue;
    const size_t ih = static_cast<size_t>(I) * H;
    // Weights in [K, N] order so the axpy inner loop is contiguous.
    std::vector<R> wg_t = transposed(w_gate + e * ih, I, H);  // [H, I]
    std::vector<R> wu_t = transposed(w_up + e * ih, I, H);    // [H, I]
    std::vector<R> wd_t = transposed(w_down + e * ih, H, I);  // [I, H]
    parallel_for(r1 - r0, [&](int64_t q) {
      const int64_t p = r0 + q;
      R* gp = g + p * I;
      R* up = u + p * I;
      R* ap = a + p * I;
      row_times_matrix<R>(x_perm + p * H, H, wg_t.data(), I, gp);
      row_times_matrix<R>(x_perm + p * H, H, wu_t.data(), I, up);
      for (int i = 0; i < I; ++i) ap[i] = gp[i] * sigmoid<R>(gp[i]) * up[i];
      row_times_matrix<R>(ap, I, wd_t.data(), H, o + p * H);
    });
  }
}

// Y[t, :] = sum over j ascending of w[t, j] * O_perm[flat_to_sorted[t*k + j], :]
template <class R>
void combine(int T, int H, int k, const R* o_perm, const R* w, const int32_t* flat_to_sorted, R* y) {
  parallel_for(T, [&](int64_t t) {
    R* yt = y + t * H;
    for (int h = 0; h < H; ++h) yt[h] = R(0);
    for (int j = 0; j < k; ++j) {
      const R wj = w[t * k + j];
      const R* op = o_perm + static_cast<int64_t>(flat_to_sorted[t * k + j]) * H;
      for (int h = 0; h < H; ++h) yt[h] = yt[h] + wj * op[h];
    }
  });
}

// ----------------------------------------------------------------------------
// Backward.
// ----------------------------------------------------------------------------

// dO_perm[p] = w[t,j] dY[t];  gw[t,j] = <dY[t], O_perm[p]>,  p = flat_to_sorted[t*k + j]
template <class R>
void combine_bwd(int T, int H, int k, const R* dy, const R* o_perm, const R* w, const int32_t* flat_to_sorted,
                 R* do_perm, R* gw) {
  parallel_for(T, [&](int64_t t) {
    const R* dyt = dy + t * H;
    for (int j = 0; j < k; ++j) {
      const int64_t p = flat_to_sorted[t * k + j];
      const R wj = w[t * k + j];
      const R* op = o_perm + p * H;
      R* dop = do_perm + p * H;
      R acc = R(0);
      for (int h = 0; h < H; ++h) {
        dop[h] = wj * dyt[h];
        acc = acc + dyt[h] * op[h];
      }
      gw[t * k + j] = acc;
    }
  });
}

// Per expert e (rows p in [offsets[e], offsets[e+1])):
//   dA = dO W_down[e]                         dW_down[e] = dO^T A
//   dU = dA * silu(G)                         dG = dA * U * s * (1 + G (1 - s)),  s = sigmoid(G)
//   dX_perm = dG W_gate[e] + dU W_up[e]       dW_gate[e] = dG^T X_perm,  dW_up[e] = dU^T X_perm
// dW of an expert with no rows is zero. expert_mask restricts the work.
template <class R>
void experts_bwd(int H, int E, int I, const R* do_perm, const R* x_perm, const R* g, const R* u, const R* a,
                 const int32_t* offsets, const R* w_gate, const R* w_up, const R* w_down,
                 const uint8_t* expert_mask, R* dx_perm, R* dw_gate, R* dw_up, R* dw_down) {
  const size_t ih = static_cast<size_t>(I) * H;
  for (int e = 0; e < E; ++e) {
    if (expert_mask && !expert_mask[e]) continue;
    const int64_t r0 = offsets[e], r1 = offsets[e + 1];
    const int64_t n = r1 - r0;
    R* dwg = dw_gate + e * ih;
    R* dwu = dw_up + e * ih;
    R* dwd = dw_down + e * ih;
    if (n <= 0) {
      for (size_t i = 0; i < ih; ++i) dwg[i] = dwu[i] = dwd[i] = R(0);
      continue;
    }
    // Row-side products: dA, dG, dU, dX_perm for every row of the expert.
    std::vector<R> dg(static_cast<size_t>(n) * I), du(static_cast<size_t>(n) * I);
    const R* wd = w_down + e * ih;  // [H, I]: already [K, N] for dA = dO W_down
    const R* wg = w_gate + e * ih;  // [I, H]: already [K, N] for dX = dG W_gate
    const R* wu = w_up + e * ih;
    parallel_for(n, [&](int64_t q) {
      const int64_t p = r0 + q;
      std::vector<R> da(I);
      row_times_matrix<R>(do_perm + p * H, H, wd, I, da.data());
      for (int i = 0; i < I; ++i) {
        const R gv = g[p * I + i], uv = u[p * I + i];
        const R s = sigmoid<R>(gv);
        du[q * I + i] = da[i] * (gv * s);
        dg[q * I + i] = da[i] * uv * s * (R(1) + gv * (R(1) - s));
      }
      // dX_perm[p] = sum over the 2I rows of [W_gate; W_up], gate part first.
      R* dxp = dx_perm + p * H;
      for (int h = 0; h < H; ++h) dxp[h] = R(0);
      for (int i = 0; i < I; ++i) {
        const R c = dg[q * I + i];
        const R* wr = wg + static_cast<size_t>(i) * H;
        for (int h = 0; h < H; ++h) dxp[h] = dxp[h] + c * wr[h];
      }
      for (int i = 0; i < I; ++i) {
        const R c = du[q * I + i];
        const R* wr = wu + static_cast<size_t>(i) * H;
        for (int h = 0; h < H; ++h) dxp[h] = dxp[h] + c * wr[h];
      }
    });
    // Weight gradients: sequential sums over the expert's rows in ascending p.
    parallel_for(H, [&](int64_t h) {  // dW_down[e][h, :] = sum_p dO[p, h] A[p, :]
      R* out = dwd + h * I;
      for (int i = 0; i < I; ++i) out[i] = R(0);
      for (int64_t q = 0; q < n; ++q) {
        const R c = do_perm[(r0 + q) * H + h];
        const R* ar = a + (r0 + q) * I;
        for (int i = 0; i < I; ++i) out[i] = out[i] + c * ar[i];
      }
    });
    parallel_for(2 * static_cast<int64_t>(I), [&](int64_t ii) {  // dW_gate / dW_up rows
      const bool up = ii >= I;
      const int64_t i = up ? ii - I : ii;
      R* out = (up ? dwu : dwg) + i * H;
      const R* d = up ? du.data() : dg.data();
      for (int h = 0; h < H; ++h) out[h] = R(0);
      for (int64_t q = 0; q < n; ++q) {
        const R c = d[q * I + i];
        const R* xr = x_perm + (r0 + q) * H;
        for (int h = 0; h < H; ++h) out[h] = out[h] + c * xr[h];
      }
    });
  }
}

// dX[t, :] = sum over j ascending of dX_perm[flat_to_sorted[t*k + j], :]
template <class R>
void unpermute_sum(int T, int H, int k, const R* dx_perm, const int32_t* flat_to_sorted, R* dx) {
  parallel_for(T, [&](int64_t t) {
    R* out = dx + t * H;
    for (int h = 0; h < H; ++h) out[h] = R(0);
    for (int j = 0; j < k; ++j) {
      const R* src = dx_perm + static_cast<int64_t>(flat_to_sorted[t * k + j]) * H;
      for (int h = 0; h < H; ++h) out[h] = out[h] + src[h];
    }
  });
}

// Gradient of the routing weights' loss contribution with respect to the
// logits, by the full chain rule through the softmax p, the kept sum S and
// the 1e-20 term:  w_j = p_{sel j} / (S + eps),  S = sum_j p_{sel j}.
//   dL/dp_i = (g_i - G) / (S + eps)  for i kept, 0 otherwise,  G = sum_j g_j w_j
//   dL/dl_e = p_e (dL/dp_e - sum_i p_i dL/dp_i)
template <class R>
void route_bwd(int T, int E, int k, const R* logits, const int32_t* idx, const R* gw, R* d_logits) {
  parallel_for(T, [&](int64_t t) {
    const R* l = logits + t * E;
    R m = l[0];
    for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
    R z = R(0);
    for (int e = 0; e < E; ++e) z = z + expo<R>(l[e] - m);
    std::vector<R> p(E), dp(E, R(0));
    for (int e = 0; e < E; ++e) p[e] = expo<R>(l[e] - m) / z;
    R s = R(0);
    for (int j = 0; j < k; ++j) s = s + p[idx[t * k + j]];
    const R den = s + R(1e-20);
    R gsum = R(0);
    for (int j = 0; j < k; ++j) gsum = gsum + gw[t * k + j] * (p[idx[t * k + j]] / den);
    for (int j = 0; j < k; ++j) dp[idx[t * k + j]] = (gw[t * k + j] - gsum) / den;
    R pdp = R(0);
    for (int e = 0; e < E; ++e) pdp = pdp + p[e] * dp[e];
    for (int e = 0; e < E; ++e) d_logits[t * E + e] = p[e] * (dp[e] - pdp);
  });
}

}  // namespace

// ----------------------------------------------------------------------------
// C entry points: _f32 (the parity reference) and _f64 (finite differences).
// Every pointer is host memory, dense row-major; indices are int32.
// ----------------------------------------------------------------------------
#define ORACLE_EXPORT extern "C" __attribute__((visibility("default")))

ORACLE_EXPORT void oracle_set_threads(int n) { g_threads = n; }
ORACLE_EXPORT int oracle_threads() { return thread_count(); }

ORACLE_EXPORT int oracle_permute_index(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                                       int32_t* sorted_to_flat, int32_t* flat_to_sorted) {
  return permute_index(T, E, k, idx, counts, offsets, sorted_to_flat, flat_to_sorted);
}

#define ORACLE_TYPED(SUF, R)                                                                                   \
  ORACLE_EXPORT int oracle_route_##SUF(int T, int H, int E, int k, const R* x, const R* wr, const R* bias,      \
                                       R* logits, int32_t* idx, R* w) {                                        \
    return route<R>(T, H, E, k, x, wr, bias, logits, idx, w);                                                 \
  }                                                                                                            \
  ORACLE_EXPORT void oracle_gather_##SUF(int T, int H, int k, const R* x, const int32_t* s2f, R* x_perm) {     \
    gather_rows<R>(T, H, k, x, s2f, x_perm);                                                                  \
  }                                                                                                            \
  ORACLE_EXPORT void oracle_experts_fwd_##SUF(int H, int E, int I, const R* x_perm, const int32_t* offsets,    \
                                              const R* wg, const R* wu, const R* wd, const uint8_t* mask,      \
                                              R* g, R* u, R* a, R* o) {                                        \
    experts_fwd<R>(H, E, I, x_perm, offsets, wg, wu, wd, mask, g, u, a, o);                                   \
  }                                                                                                            \
  ORACLE_EXPORT void oracle_combine_##SUF(int T, int H, int k, const R* o_perm, const R* w, const int32_t* f2s, \
                                          R* y) {                                                              \
    combine<R>(T, H, k, o_perm, w, f2s, y);                                                                   \
  }                                                                                                            \
  ORACLE_EXPORT void oracle_combine_bwd_##SUF(int T, int H, int k, const R* dy, const R* o_perm, const R* w,   \
                                              const int32_t* f2s, R* do_perm, R* gw) {                         \
    combine_bwd<R>(T, H, k, dy, o_perm, w, f2s, do_perm, gw);                                                 \
  }                                                                                                            \
  ORACLE_EXPORT void oracle_experts_bwd_##SUF(int H, int E, int I, const R* do_perm, const R* x_perm,          \
                                              const R* g, const R* u, const R* a, const int32_t* offsets,      \
                                              const R* wg, const R* wu, const R* wd, const uint8_t* mask,      \
                                              R* dx_perm, R* dwg, R* dwu, R* dwd) {                            \
    experts_bwd<R>(H, E, I, do_perm, x_perm, g, u, a, offsets, wg, wu, wd, mask, dx_perm, dwg, dwu, dwd);     \
  }                                                                                                            \
  ORACLE_EXPORT void oracle_unpermute_sum_##SUF(int T, int H, int k, const R* dx_perm, const int32_t* f2s,     \
                                                R* dx) {                                                       \
    unpermute_sum<R>(T, H, k, dx_perm, f2s, dx);                                                              \
  }                                                                                                            \
  ORACLE_EXPORT void oracle_route_bwd_##SUF(int T, int E, int k, const R* logits, const int32_t* idx,         \
                                            const R* gw, R* d_logits) {                                       \
    route_bwd<R>(T, E, k, logits, idx, gw, d_logits);                                                         \
  }

ORACLE_TYPED(f32, float)
ORACLE_TYPED(f64, double)
