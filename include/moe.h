/* moe.h — C ABI of the fused MoE expert stage for MI355X (gfx950).
 *
 * One MoE layer's expert stage on one GPU, forward and backward, as a chain of
 * calls on one HIP stream:
 *
 *   forward : moe_route -> moe_permute -> moe_grouped_gemm_fwd -> moe_combine
 *   backward: moe_combine_bwd -> moe_grouped_gemm_bwd -> moe_unpermute_sum -> moe_route_bwd
 *   inference (gather and routing weights fused into the GEMMs):
 *             moe_forward_fused = moe_route -> moe_permute_fused ->
 *             moe_gemm_gate_up_gathered -> moe_gemm_down_weighted -> moe_unpermute_sum
 *   fp8 inference: moe_forward_fused_fp8 = moe_route -> moe_permute_fused ->
 *             moe_quantize_fp8_rows (x) -> moe_gemm_gate_up_fp8 ->
 *             moe_quantize_fp8_rows (a) -> moe_gemm_down_fp8 -> moe_unpermute_sum
 *             (moe_forward_fused_mxfp4: the same with MXFP4 weights)
 *   training without do_perm: moe_route -> moe_permute_rows ->
 *             moe_gemm_gate_up_aw -> moe_gemm_down -> moe_combine;
 *             moe_combine_bwd (do_perm NULL) -> moe_gemm_down_bwd_dy ->
 *             moe_gemm_gate_up_bwd -> moe_unpermute_sum -> moe_route_bwd
 *   training without x_perm (the gather fused into both GEMMs that read x):
 *             moe_route -> moe_permute_fused -> moe_gemm_gate_up_gathered ->
 *             moe_gemm_down -> moe_combine; moe_combine_bwd -> moe_gemm_down_dgrad,
 *             moe_gemm_down_wgrad, moe_gemm_gate_up_dgrad,
 *             moe_gemm_gate_up_wgrad_gathered -> moe_unpermute_sum -> moe_route_bwd
 *   adapters on frozen experts: moe_lora_merge -> the forward on the merged
 *             weights; moe_combine_bwd -> moe_gemm_down_dgrad ->
 *             moe_gemm_gate_up_dgrad -> moe_unpermute_sum -> moe_route_bwd,
 *             moe_lora_grads
 *
 * It replaces the per-expert for-loop of the Hugging Face MoE block (axolotl
 * issue #3155, "Feature description") with router softmax/top-k, a sort of the
 * (token, expert) pairs by expert, grouped GEMMs over the stacked expert
 * weights with a SwiGLU epilogue, and a weighted combine (sourcepulse summary
 * of the Triton fused-MoE repository, "How It Works").
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer (hipMalloc'd or a torch CUDA
 *     tensor's data_ptr), to a dense row-major array.
 *   - Indices are int32. T*k must stay below 2^31.
 *   - Activations and weights (x, w_*, g, u, a, o_perm, y, dy, do_perm,
 *     dx_perm, dx) have element type shape.dtype: MOE_F32 (float) or MOE_BF16
 *     (bfloat16 bit patterns). Router outputs (logits, topk_w, d_topk_w,
 *     d_logits) and weight gradients (dw_*) are always float32.
 *   - The caller owns every buffer, including the workspace; the library never
 *     allocates device memory and keeps no pointer after a call returns.
 *   - Each call only enqueues kernels on `stream` and returns; it never
 *     synchronises. Outputs are fully overwritten (except dw_* with
 *     accumulate_dw = 1). Results are deterministic: no floating-point
 *     atomics, so reruns are bitwise identical.
 *   - Errors: every argument is checked on the host before any HIP call; a
 *     bad argument returns MOE_EINVAL (null pointer, non-positive size, k > E,
 *     E > 1024, T*k >= 2^31), MOE_EUNSUPPORTED (H or I not a multiple of 64,
 *     unknown dtype) or MOE_EWORKSPACE (workspace too small), with nothing
 *     enqueued. A failed launch returns MOE_EHIP. Faults inside kernels
 *     surface at the caller's next synchronisation. No C++ exception crosses
 *     this interface.
 *   - Calls on disjoint buffers may run concurrently on different streams.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,
  MOE_EUNSUPPORTED = 2,
  MOE_EWORKSPACE = 3,
  MOE_EHIP = 4
} moe_status;

/* T tokens, hidden size H, E experts, k experts per token, expert
 * intermediate size I; dtype is a moe_dtype. */
typedef struct {
  int32_t T, H, E, k, I;
  int32_t dtype;
} moe_shape;

/* Bytes of device workspace for this shape on the current device. One
 * buffer of this size serves every call that takes a workspace:
 * moe_permute's per-block expert histograms, moe_grouped_gemm_bwd's dG and
 * dU for every row ([T*k, 2I] in dtype), and (bf16) the weight gradients'
 * split-K partial tiles: an expert whose row count is far above a CU's share
 * of the launch is reduced in chunks whose fp32 partial 256 x 256 tiles are
 * added in chunk order afterwards (deterministic; at most two tiles per
 * compute unit, 128 MiB on a 256-CU device, fewer for small shapes). */
size_t moe_workspace_bytes(moe_shape s);

/* Router (torchtune PR #2820 "[WIP] Qwen3 MoE support", comment on dividing
 * the top scores by their sum plus 1e-20; axolotl issue #3155, comments on
 * the router weight shape; sourcepulse summary, "Highlighted Details": fused
 * softmax + top-k).
 *   x [T,H], w_router [E,H] (nn.Linear(H, E) layout), logit_bias [E] float32
 *   or NULL.
 *   logits[t,e] = fp32 fma chain over h ascending from +0, then + bias[e];
 *   topk_idx[t,:] = the k largest logits, largest first, ties to the lower
 *   expert index; a NaN logit ranks below every number, -inf included (so
 *   every index is a valid expert whatever the logits); topk_w[t,j] =
 *   p[idx] / (sum_j p[idx] + 1e-20) with p = softmax(logits[t,:]) in fp32 (NaN
 *   for a token with a NaN logit).
 * Outputs: logits [T,E] f32, topk_idx [T,k] int32, topk_w [T,k] f32. */
moe_status moe_route(moe_shape s, const void* x, const void* w_router, const float* logit_bias,
                     float* logits, int32_t* topk_idx, float* topk_w, hipStream_t stream);

/* Expert indexing and gather (unsloth PR #3812 "[MoE] Improve moe kernels",
 * review suggestion: counts by bincount, the order by a stable argsort of
 * the flattened expert ids).
 *   counts[e] = #{f : topk_idx[f] == e} (shape [E]), offsets [E+1] its
 *   exclusive prefix sum; for flat index f = t*k + j,
 *   flat_to_sorted[f] = offsets[e_f] + #{f' < f : e_f' == e_f},
 *   sorted_to_flat is its inverse; x_perm[p,:] = x[sorted_to_flat[p] / k, :].
 *   topk_idx values must lie in [0, E) (not checked on the device).
 * Outputs: counts [E], offsets [E+1], sorted_to_flat [T*k],
 * flat_to_sorted [T*k] (int32), x_perm [T*k,H]. Workspace: ws of ws_bytes >=
 * moe_workspace_bytes(s). */
moe_status moe_permute(moe_shape s, const int32_t* topk_idx, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_to_flat, int32_t* flat_to_sorted, void* x_perm,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Grouped GEMMs of the forward over the expert-sorted rows (sourcepulse
 * summary, "How It Works": grouped GEMM on inputs sorted by expert; unsloth
 * PR #3812, stacked gate/up [E,2I,H] and down [E,H,I] weights, held here as
 * separate W_gate and W_up; axolotl issue #3155, numerical-check comment:
 * silu gating, no bias). For each expert e and row p in
 * [offsets[e], offsets[e+1]):
 *   g = x_perm[p] W_gate[e]^T, u = x_perm[p] W_up[e]^T, a = silu(g) * u,
 *   o_perm[p] = a W_down[e]^T      (fp32 accumulation; stored in dtype).
 * Inputs: x_perm [T*k,H], offsets [E+1] (device, from moe_permute),
 * w_gate, w_up [E,I,H], w_down [E,H,I]. Outputs: g, u, a [T*k,I] (kept for
 * the backward), o_perm [T*k,H]. ws/ws_bytes are accepted for interface
 * symmetry and may be NULL/0. */
moe_status moe_grouped_gemm_fwd(moe_shape s, const void* x_perm, const int32_t* offsets, const void* w_gate,
                                const void* w_up, const void* w_down, void* g, void* u, void* a, void* o_perm,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* The six grouped GEMMs one at a time (moe_grouped_gemm_fwd chains the
 * first two; moe_grouped_gemm_bwd runs the other four as the two paired
 * launches below, with the same results). Same operands, layouts and arithmetic as
 * described there; dgu is [T*k, 2I] in dtype holding dG in columns [0, I)
 * and dU in columns [I, 2I). Callers that train adapters on frozen experts
 * can run the data gradients without the weight gradients.
 *   moe_gemm_gate_up       g, u, a  <- x_perm, W_gate, W_up
 *   moe_gemm_down          o_perm   <- a, W_down
 *   moe_gemm_down_dgrad    dgu      <- do_perm, W_down, g, u
 *   moe_gemm_down_wgrad    dw_down  <- do_perm, a              (f32; += if accumulate_dw)
 *   moe_gemm_gate_up_dgrad dx_perm  <- dgu, W_gate, W_up
 *   moe_gemm_gate_up_wgrad dw_gate, dw_up <- dgu, x_perm       (f32; += if accumulate_dw)
 * The two weight-gradient calls take the workspace (ws_bytes >=
 * moe_workspace_bytes(s), else MOE_EWORKSPACE) for their split-K partial
 * tiles; calls that share one workspace must not overlap in time. */
moe_status moe_gemm_gate_up(moe_shape s, const void* x_perm, const int32_t* offsets, const void* w_gate,
                            const void* w_up, void* g, void* u, void* a, hipStream_t stream);
moe_status moe_gemm_down(moe_shape s, const void* a, const int32_t* offsets, const void* w_down, void* o_perm,
                         hipStream_t stream);
moe_status moe_gemm_down_dgrad(moe_shape s, const void* do_perm, const int32_t* offsets, const void* w_down,
                               const void* g, const void* u, void* dgu, hipStream_t stream);
moe_status moe_gemm_down_wgrad(moe_shape s, const void* do_perm, const void* a, const int32_t* offsets,
                               float* dw_down, int accumulate_dw, void* ws, size_t ws_bytes, hipStream_t stream);
moe_status moe_gemm_gate_up_dgrad(moe_shape s, const void* dgu, const int32_t* offsets, const void* w_gate,
                                  const void* w_up, void* dx_perm, hipStream_t stream);
moe_status moe_gemm_gate_up_wgrad(moe_shape s, const void* dgu, const void* x_perm, const int32_t* offsets,
                                  float* dw_gate, float* dw_up, int accumulate_dw, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* Weighted combine (modelopt.torch.utils.moe, a2a_moe: each token's k expert
 * results are weighted by its routing weights in their own precision and
 * summed; the result returns in the hidden dtype).
 *   y[t,:] = sum over j ascending of topk_w[t,j] * o_perm[flat_to_sorted[t*k+j],:]
 *   in fp32, rounded once to dtype. Output: y [T,H]. */
moe_status moe_combine(moe_shape s, const void* o_perm, const float* topk_w, const int32_t* flat_to_sorted,
                       void* y, hipStream_t stream);

/* Backward of moe_combine (chain rule of the combine above).
 *   do_perm[p,:] = topk_w[t,j] * dy[t,:], d_topk_w[t,j] = <dy[t,:], o_perm[p,:]>
 *   with p = flat_to_sorted[t*k+j]. Outputs: do_perm [T*k,H] (dtype),
 *   d_topk_w [T,k] f32. do_perm may be NULL: only d_topk_w is written (the
 *   backward of moe_gemm_down_bwd_dy reads dy itself). */
moe_status moe_combine_bwd(moe_shape s, const void* dy, const void* o_perm, const float* topk_w,
                           const int32_t* flat_to_sorted, void* do_perm, float* d_topk_w, hipStream_t stream);

/* Backward of moe_grouped_gemm_fwd (chain rule of the expert MLP above). For
 * each expert e, over its rows:
 *   dA = do_perm W_down[e];  dU = dA * silu(g);  dG = dA * u * s * (1 + g (1 - s)), s = sigmoid(g)
 *   dx_perm = dG W_gate[e] + dU W_up[e]
 *   dW_down[e] = do_perm^T a,  dW_gate[e] = dG^T x_perm,  dW_up[e] = dU^T x_perm
 * Weight gradients are float32 with fp32 accumulation; an expert with no rows
 * gets zeros. accumulate_dw = 0 overwrites dw_*, 1 adds to them.
 * Inputs as produced by the forward. Outputs: dx_perm [T*k,H] (dtype),
 * dw_gate, dw_up [E,I,H] f32, dw_down [E,H,I] f32. Workspace: ws of
 * ws_bytes >= moe_workspace_bytes(s). */
moe_status moe_grouped_gemm_bwd(moe_shape s, const void* do_perm, const void* x_perm, const void* g,
                                const void* u, const void* a, const int32_t* offsets, const void* w_gate,
                                const void* w_up, const void* w_down, void* dx_perm, float* dw_gate,
                                float* dw_up, float* dw_down, int accumulate_dw, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* The backward's GEMMs in two launches (moe_grouped_gemm_bwd chains these):
 * each runs a data gradient and then the weight gradient that reads the
 * same inputs in one persistent launch, so that a workgroup done with the
 * first starts on the second without waiting for the first's slowest one.
 * Results are the same bits as the single-GEMM calls above.
 *   moe_gemm_down_bwd     dgu <- do_perm, W_down, g, u  and  dw_down <- do_perm, a
 *   moe_gemm_gate_up_bwd  dx_perm <- dgu, W_gate, W_up  and  dw_gate, dw_up <- dgu, x rows
 * x rows: x_perm when row_token is NULL; otherwise x [T,H] with sorted row p
 * read as row row_token[p] (from moe_permute_fused; the limits of
 * moe_gemm_gate_up_wgrad_gathered apply). dw_* f32 (+= if accumulate_dw).
 * Workspace: ws of ws_bytes >= moe_workspace_bytes(s) (split-K partials of
 * the weight gradient). */
moe_status moe_gemm_down_bwd(moe_shape s, const void* do_perm, const void* a, const int32_t* offsets,
                             const void* w_down, const void* g, const void* u, void* dgu, float* dw_down,
                             int accumulate_dw, void* ws, size_t ws_bytes, hipStream_t stream);
moe_status moe_gemm_gate_up_bwd(moe_shape s, const void* dgu, const void* x_rows, const int32_t* row_token,
                                const int32_t* offsets, const void* w_gate, const void* w_up, void* dx_perm,
                                float* dw_gate, float* dw_up, int accumulate_dw, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* ---- Training step without do_perm (unsloth PR #3812, "[MoE] Improve moe
 * kernels for unsloth fine tuning", Codex review of the grouped GEMM's
 * fused routing-weight multiply; modelopt.torch.utils.moe, a2a_moe: each
 * token's expert outputs weighted by its routing weights). The backward of
 * the weighted combine no longer materialises do_perm = w * dy per sorted
 * row: the down data gradient reads dy rows through the rows' tokens and
 * applies the routing weight to dA in fp32, and the down weight gradient
 * reads the same dy rows against the weighted activations a_w = w * a that
 * the forward's gate/up GEMM writes. Chain (bf16 only): moe_route ->
 * moe_permute_rows -> moe_gemm_gate_up_aw -> moe_gemm_down -> moe_combine;
 * moe_combine_bwd (do_perm NULL) -> moe_gemm_down_bwd_dy ->
 * moe_gemm_gate_up_bwd -> moe_unpermute_sum -> moe_route_bwd. */

/* moe_permute with, for each sorted row p, row_token[p] = sorted_to_flat[p] / k
 * (int32 [T*k]) and row_weight[p] = topk_w[sorted_to_flat[p]] (f32 [T*k]) as
 * in moe_permute_fused; every other output (counts, offsets, both
 * permutations, x_perm) exactly as moe_permute. */
moe_status moe_permute_rows(moe_shape s, const int32_t* topk_idx, const float* topk_w, const void* x,
                            int32_t* counts, int32_t* offsets, int32_t* sorted_to_flat, int32_t* flat_to_sorted,
                            int32_t* row_token, float* row_weight, void* x_perm, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* moe_gemm_gate_up that also writes the weighted activations
 *   a_w[p,:] = bf16(row_weight[p] * a[p,:])  (a in fp32 before its rounding)
 * for moe_gemm_down_bwd_dy. x_rows is x_perm [T*k,H] when row_token is NULL,
 * else x [T,H] with sorted row p read as row row_token[p] (then
 * T*H*2 < 2^31, MOE_EUNSUPPORTED otherwise). g, u, a, a_w [T*k,I] bf16;
 * shape.dtype MOE_BF16 (MOE_EUNSUPPORTED otherwise). */
moe_status moe_gemm_gate_up_aw(moe_shape s, const void* x_rows, const int32_t* row_token, const float* row_weight,
                               const int32_t* offsets, const void* w_gate, const void* w_up, void* g, void* u,
                               void* a, void* a_w, hipStream_t stream);

/* The down backward pair (moe_gemm_down_bwd) reading dy [T,H] through the
 * rows' tokens instead of do_perm. For each expert e and sorted row p of it,
 * t = row_token[p], w = row_weight[p]:
 *   dA[p] = w * (dy[t] W_down[e])   (fp32; then dU, dG into dgu as in moe_gemm_down_bwd)
 *   dW_down[e] = sum over p of dy[t]^T a_w[p]   (a_w from moe_gemm_gate_up_aw)
 * which is the chain rule through do_perm[p] = w dy[t] with the weight moved
 * to the other factor (rounded once to bf16 with a, instead of with dy).
 * dgu [T*k,2I] bf16, dw_down [E,H,I] f32 (+= if accumulate_dw); workspace as
 * moe_gemm_down_bwd. bf16 only; T*H*2 < 2^31 and 4*(T*k + 256) < 2^31
 * (MOE_EUNSUPPORTED otherwise). */
moe_status moe_gemm_down_bwd_dy(moe_shape s, const void* dy, const int32_t* row_token, const float* row_weight,
                                const void* a_w, const int32_t* offsets, const void* w_down, const void* g,
                                const void* u, void* dgu, float* dw_down, int accumulate_dw, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* Backward of the gather in moe_permute: dx[t,:] = sum over j ascending of
 * dx_perm[flat_to_sorted[t*k+j],:] in fp32, rounded once. Output: dx [T,H]. */
moe_status moe_unpermute_sum(moe_shape s, const void* dx_perm, const int32_t* flat_to_sorted, void* dx,
                             hipStream_t stream);

/* Backward of the routing weights (chain rule of the renormalised top-k
 * softmax in moe_route):
 *   d_logits[t,e] = w_j (g_j - sum_i w_i g_i) if e = topk_idx[t,j], else 0,
 *   with w = topk_w and g = d_topk_w. (The exact derivative also carries terms
 *   of relative size 1e-20 from the renormalisation constant; they are
 *   dropped.) An index outside [0, E) contributes nothing (its slot still
 *   counts in the sum). Output: d_logits [T,E] f32. */
moe_status moe_route_bwd(moe_shape s, const float* d_topk_w, const float* topk_w, const int32_t* topk_idx,
                         float* d_logits, hipStream_t stream);

/* ---- Inference forward with the gather and the routing weights fused into
 * the GEMMs (the fused-mul-post path of unsloth PR #3812, "[MoE] Improve moe
 * kernels for unsloth fine tuning", Codex review of the grouped GEMM
 * interface; the unsorted-token gather of the sourcepulse summary, "How It
 * Works"). No x_perm is built and no weighted combine runs: the gate/up GEMM
 * reads each sorted row straight from x, the down GEMM multiplies each output
 * row by its routing weight before rounding, and y is the plain per-token sum
 * of moe_unpermute_sum. The result equals moe_route -> moe_permute ->
 * moe_grouped_gemm_fwd -> moe_combine up to where the rounding to the
 * activation dtype happens (here after the weight is applied). */

/* moe_permute without the gather: counts, offsets, sorted_to_flat and
 * flat_to_sorted exactly as moe_permute, plus for each sorted row p
 *   row_token[p]  = sorted_to_flat[p] / k          (int32 [T*k])
 *   row_weight[p] = topk_w[sorted_to_flat[p]]      (f32   [T*k])
 * Inputs: topk_idx [T,k] int32, topk_w [T,k] f32 (from moe_route).
 * Workspace: ws of ws_bytes >= moe_workspace_bytes(s). */
moe_status moe_permute_fused(moe_shape s, const int32_t* topk_idx, const float* topk_w, int32_t* counts,
                             int32_t* offsets, int32_t* sorted_to_flat, int32_t* flat_to_sorted, int32_t* row_token,
                             float* row_weight, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_gemm_gate_up with row p of its input read as row row_token[p] of x
 * [T,H] (dtype) instead of x_perm. g and u [T*k,I] are stored when both are
 * non-null, skipped when both are null (inference needs a only); one null and
 * one not is MOE_EINVAL. T*H*sizeof(dtype) must stay below 2^31
 * (MOE_EUNSUPPORTED otherwise). */
moe_status moe_gemm_gate_up_gathered(moe_shape s, const void* x, const int32_t* row_token, const int32_t* offsets,
                                     const void* w_gate, const void* w_up, void* g, void* u, void* a,
                                     hipStream_t stream);

/* moe_gemm_down with output row p multiplied by row_weight[p] (f32, from
 * moe_permute_fused) in fp32 before the rounding to dtype:
 *   o_perm[p,:] = row_weight[p] * (a[p,:] W_down[e]^T). */
moe_status moe_gemm_down_weighted(moe_shape s, const void* a, const int32_t* offsets, const void* w_down,
                                  const float* row_weight, void* o_perm, hipStream_t stream);

/* moe_gemm_gate_up_wgrad with k-row p of its x operand read as row
 * row_token[p] of x [T,H] (dtype) instead of x_perm, so that training needs
 * no x_perm either (row_token from moe_permute_fused):
 *   dw_gate[e] = dG_e^T X_e,  dw_up[e] = dU_e^T X_e,  X_e[p,:] = x[row_token[p],:]
 * over the rows p of expert e. Same outputs, workspace and accumulate_dw
 * rules as moe_gemm_gate_up_wgrad. T*H*sizeof(dtype) and 4*(T*k + 256) must
 * stay below 2^31 (MOE_EUNSUPPORTED otherwise). */
moe_status moe_gemm_gate_up_wgrad_gathered(moe_shape s, const void* dgu, const void* x, const int32_t* row_token,
                                           const int32_t* offsets, float* dw_gate, float* dw_up, int accumulate_dw,
                                           void* ws, size_t ws_bytes, hipStream_t stream);

/* The fused inference forward in one call: moe_route (logits, topk_idx,
 * topk_w), moe_permute_fused (counts, offsets, sorted_to_flat,
 * flat_to_sorted, row_token, row_weight), moe_gemm_gate_up_gathered (a only),
 * moe_gemm_down_weighted (o_perm) and moe_unpermute_sum (y [T,H]). Every
 * buffer is caller-owned and overwritten; logit_bias may be NULL. Workspace:
 * ws of ws_bytes >= moe_workspace_bytes(s). */
moe_status moe_forward_fused(moe_shape s, const void* x, const void* w_router, const float* logit_bias,
                             const void* w_gate, const void* w_up, const void* w_down, float* logits,
                             int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                             int32_t* sorted_to_flat, int32_t* flat_to_sorted, int32_t* row_token, float* row_weight,
                             void* a, void* o_perm, void* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_forward_fused for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * calls and results, bit for bit, with no workspace argument. The sort's
 * per-block histograms (ceil(T*k / 1024) * E int32) live instead in a static
 * device array of the library, 4 MiB per device, held by each device the
 * library runs on until the process ends; a larger shape returns
 * MOE_EWORKSPACE with nothing enqueued. The function allocates nothing. Every
 * call on a device shares that device's array, so calls that overlap in time
 * on one device (concurrent streams, other host threads) race and must be
 * ordered by the caller. */
moe_status moe_forward_fused_noalloc(moe_shape s, const void* x, const void* w_router, const float* logit_bias,
                                     const void* w_gate, const void* w_up, const void* w_down, float* logits,
                                     int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                                     int32_t* sorted_to_flat, int32_t* flat_to_sorted, int32_t* row_token,
                                     float* row_weight, void* a, void* o_perm, void* y, hipStream_t stream);

/* ---- fp8 inference forward (the quantised expert weights of the sourcepulse
 * summary: bitsandbytes 4-bit compatibility, "Quick Start & Requirements";
 * QLoRA and training over quantised GGUF models, "Highlighted Details"; the
 * fused 4-bit dequantisation, "Limitations & Caveats"; and the question on
 * fp8 checkpoints in torchtune PR #2820; taken to the 8-bit floats gfx950's
 * matrix cores multiply natively). Both GEMM operands are
 * OCP E4M3 codes (bias 7, largest finite 448, 0x7F/0xFF NaN); every row of
 * an operand carries one power-of-two scale as an E8M0 byte c (2^(c-127)).
 * The GEMMs multiply codes and apply both scales inside the matrix core, so
 * a product is exactly dequant(a) * dequant(w), summed in fp32. */

/* Rows [rows, K] of bf16 -> E4M3 codes q [rows, K] and one scale per row.
 * Scale 2^X with X the smallest integer for which max |row| / 2^X <= 448,
 * clamped to [-127, 127] (-127 for an all-zero row), so that no element is
 * clipped; q = E4M3(clamp(x / 2^X, -448, 448)), rounded to nearest, ties to
 * even. e8 layout: [rows] when flat_to_sorted is NULL;
 * otherwise [rows * k] in sorted order, row r's scale written at
 * flat_to_sorted[r * k + j] for every j < k (x's scales for the gathered
 * gate/up GEMM). K % 8 == 0 (MOE_EINVAL otherwise). Weights are quantised
 * once with the same call: w_gate, w_up [E,I,H] as E*I rows, w_down [E,H,I]
 * as E*H rows (one scale per output channel). */
moe_status moe_quantize_fp8_rows(int32_t rows, int32_t K, const void* in, uint8_t* q, uint8_t* e8,
                                 const int32_t* flat_to_sorted, int32_t k, hipStream_t stream);

/* Gathered gate/up GEMM in fp8 with the SwiGLU epilogue, storing a only:
 *   a[p,:] = bf16(silu(g) * u),  g = deq(xq[row_token[p]]) deq(Wg[e])^T,  u likewise
 * xq [T,H] codes with x_e8 [T*k] (sorted order, from moe_quantize_fp8_rows
 * with flat_to_sorted); wq_gate, wq_up [E,I,H] with w_gate_e8, w_up_e8
 * [E,I]; a [T*k,I] bf16. Requires shape.dtype MOE_BF16, H and I multiples of
 * 64 and T*H < 2^31 (MOE_EUNSUPPORTED otherwise). */
moe_status moe_gemm_gate_up_fp8(moe_shape s, const uint8_t* xq, const uint8_t* x_e8, const int32_t* row_token,
                                const int32_t* offsets, const uint8_t* wq_gate, const uint8_t* w_gate_e8,
                                const uint8_t* wq_up, const uint8_t* w_up_e8, void* a, hipStream_t stream);

/* Weighted down GEMM in fp8:
 *   o_perm[p,:] = bf16(row_weight[p] * deq(aq[p]) deq(Wd[e])^T)
 * aq [T*k,I] codes with a_e8 [T*k]; wq_down [E,H,I] with w_down_e8 [E,H];
 * o_perm [T*k,H] bf16. Same shape limits as moe_gemm_gate_up_fp8. */
moe_status moe_gemm_down_fp8(moe_shape s, const uint8_t* aq, const uint8_t* a_e8, const int32_t* offsets,
                             const uint8_t* wq_down, const uint8_t* w_down_e8, const float* row_weight, void* o_perm,
                             hipStream_t stream);

/* The fp8 inference forward in one call: moe_route, moe_permute_fused,
 * moe_quantize_fp8_rows (x -> xq [T,H], x_e8 [T*k] sorted),
 * moe_gemm_gate_up_fp8 (a [T*k,I] bf16), moe_quantize_fp8_rows (a -> aq
 * [T*k,I], a_e8 [T*k]), moe_gemm_down_fp8 (o_perm) and moe_unpermute_sum
 * (y [T,H]). Weights come quantised. Every buffer is caller-owned;
 * logit_bias may be NULL; ws of ws_bytes >= moe_workspace_bytes(s). */
moe_status moe_forward_fused_fp8(moe_shape s, const void* x, const void* w_router, const float* logit_bias,
                                 const uint8_t* wq_gate, const uint8_t* w_gate_e8, const uint8_t* wq_up,
                                 const uint8_t* w_up_e8, const uint8_t* wq_down, const uint8_t* w_down_e8,
                                 float* logits, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                                 int32_t* sorted_to_flat, int32_t* flat_to_sorted, int32_t* row_token,
                                 float* row_weight, uint8_t* xq, uint8_t* x_e8, void* a, uint8_t* aq, uint8_t* a_e8,
                                 void* o_perm, void* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* Low-rank adapters on the frozen experts (sourcepulse summary, "Highlighted
 * Details": LoRA and QLoRA on the fused experts; torchtune PR #2820: LoRA
 * support for the Qwen3 MoE port). Adapters come in the fused format, one
 * stacked tensor per projection over all experts. Per expert e
 * and projection P in {gate, up, down} with frozen W_P [E,N,K] (w_gate, w_up
 * [E,I,H]; w_down [E,H,I]), adapters A_P [E,r,K] and B_P [E,N,r] (bf16) and
 * scale s, the stage is the plain one on W'_P = W_P + s B_P A_P. Training:
 *   moe_lora_merge (three times) -> the forward chain on W' ->
 *   moe_combine_bwd -> moe_gemm_down_dgrad -> moe_gemm_gate_up_dgrad ->
 *   moe_unpermute_sum -> moe_route_bwd, and moe_lora_grads for the adapters
 * (the frozen weights take no gradient). Rank r: a multiple of 8, at most
 * 128 (MOE_EUNSUPPORTED otherwise; r <= 0 is MOE_EINVAL). */

/* W'[e] = bf16(W[e] + s * B[e] A[e]) for w [E,N,K], a [E,r,K], b [E,N,r],
 * w_out [E,N,K], all bf16: the product summed in fp32 from exact bf16
 * products, scaled and added in fp32, rounded once. w_out may be w (in
 * place); otherwise the two must not overlap. K % 8 == 0, E <= 65535 and
 * (N + 256) K < 2^30 (MOE_EUNSUPPORTED otherwise). */
moe_status moe_lora_merge(int32_t E, int32_t N, int32_t K, int32_t r, float scale, const void* w, const void* a,
                          const void* b, void* w_out, hipStream_t stream);

/* QLoRA-style adapters over 8-bit frozen experts (sourcepulse summary,
 * "Highlighted Details": QLoRA, LoRA training over quantised GGUF models;
 * "Quick Start & Requirements": bitsandbytes 4-bit weights; torchtune PR
 * #2820: fp8 checkpoints). The frozen weights stay in E4M3 with one E8M0
 * scale per output row (moe_quantize_fp8_rows), half the bytes of bf16; the
 * merge dequantises them (exactly) and adds the adapters' product:
 *   W'[e] = bf16(deq(wq[e]) + s * B[e] A[e]),  deq(wq)[n,c] = E4M3(wq[n,c]) * 2^(w_e8[n] - 127)
 * wq [E,N,K] codes, w_e8 [E,N] (one byte per row of every expert), a, b,
 * w_out as in moe_lora_merge (w_out bf16 [E,N,K], not overlapping wq). The
 * rest of the adapter step runs on W' exactly as with bf16 frozen weights.
 * Same limits and errors as moe_lora_merge. */
moe_status moe_lora_merge_fp8(int32_t E, int32_t N, int32_t K, int32_t r, float scale, const uint8_t* wq,
                              const uint8_t* w_e8, const void* a, const void* b, void* w_out, hipStream_t stream);

/* Adapters over 4-bit frozen experts (sourcepulse summary, "Highlighted
 * Details": QLoRA over 4-bit bases; "Quick Start & Requirements":
 * bitsandbytes 4-bit weights), in the 4-bit format native to gfx950: the
 * OCP microscaling FP4 (MXFP4). Elements are E2M1 (sign, 2 exponent bits
 * with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two
 * per byte with the even element in the low nibble; every 32 consecutive
 * elements of a row share one E8M0 scale byte c (2^(c - 127)).
 *
 * moe_quantize_mxfp4_rows: rows [rows, K] of bf16 (K % 32 == 0, else
 * MOE_EINVAL) -> codes q [rows, K/2] and scales e8 [rows, K/32]. A block's
 * scale is 2^X with X the smallest integer for which max |block| / 2^X <= 6,
 * clamped to [-127, 127] (-127 for an all-zero block), so nothing is
 * clipped; each element is x / 2^X rounded to the nearest E2M1 magnitude,
 * ties to the even mantissa, with x's sign (a negative value that rounds to
 * zero is a negative zero). Inputs must be finite. */
moe_status moe_quantize_mxfp4_rows(int32_t rows, int32_t K, const void* in, uint8_t* q, uint8_t* e8,
                                   hipStream_t stream);

/* W'[e] = bf16(deq(wq[e]) + s * B[e] A[e]) over MXFP4 frozen weights: wq
 * [E,N,K/2] codes and w_e8 [E,N,K/32] scales as moe_quantize_mxfp4_rows
 * writes them for the E*N rows of a stacked weight; deq exact in fp32. a, b,
 * w_out as in moe_lora_merge. K % 32 == 0 and the limits of moe_lora_merge
 * (MOE_EUNSUPPORTED otherwise). */
moe_status moe_lora_merge_mxfp4(int32_t E, int32_t N, int32_t K, int32_t r, float scale, const uint8_t* wq,
                                const uint8_t* w_e8, const void* a, const void* b, void* w_out, hipStream_t stream);

/* The adapter step without merged weights (sourcepulse summary, "Highlighted
 * Details": LoRA on the fused experts; torchtune PR #2820: LoRA for the
 * Qwen3 MoE port). The frozen W_P stay as they are and no W' is built: each
 * GEMM runs over a reduction extended by the adapter's rank,
 *   G = [X | X (sA_gate)^T] [W_gate | B_gate]^T    (U likewise, A = silu(G) U)
 *   O = [A | A (sA_down)^T] [W_down | B_down]^T
 *   dA = [dO | dO (sB_down)] [W_down; A_down]      (then the SwiGLU backward)
 *   dX_perm = [dG | dU | dG (sB_gate) | dU (sB_up)] [W_gate; W_up; A_gate; A_up]
 * which equals the stage on W' = W + s B A up to rounding: the rank-wide row
 * projections are rounded to bf16 before the GEMM, where the merged path
 * rounds W'. The projections stay in the workspace and give the adapter
 * gradients without a second pass (moe_lora_grads_unmerged). The chain, all
 * on one stream:
 *   moe_lora_prepare (once per step: the adapters, scaled and stacked) ->
 *   moe_route -> moe_permute -> moe_lora_gemm_gate_up -> moe_lora_gemm_down ->
 *   moe_combine; moe_combine_bwd -> moe_lora_gemm_down_dgrad ->
 *   moe_lora_gemm_gate_up_dgrad -> moe_unpermute_sum -> moe_route_bwd, and
 *   moe_lora_grads_unmerged.
 * Every call takes the rank r (as moe_lora_grads: a multiple of 8, at most
 * 128), the workspace ws of ws_bytes >= moe_lora_unmerged_workspace_bytes
 * (MOE_EWORKSPACE otherwise; it holds the stacks and the projections
 * between the calls, so the calls of one step must not overlap another
 * step's) and the shapes and buffers of the plain call it replaces. The
 * projections' rows are addressed with 32-bit byte offsets: T*k*4*rp < 2^31,
 * rp = r rounded up to 32, 64 or 128 (MOE_EUNSUPPORTED otherwise). */

/* Bytes of workspace for the unmerged adapter step (0 if shape or rank are
 * rejected): the regions of moe_lora_workspace_bytes (the scaled stacks,
 * the projections, the outer products' plan and partial tiles). The GEMMs'
 * extensions read the adapters themselves, padded with zeros to rp inside
 * the kernel. */
size_t moe_lora_unmerged_workspace_bytes(moe_shape s, int32_t r);

/* The adapters of this step (a_P [E,r,K], b_P [E,N,r] bf16, scale s) into
 * ws: the scaled stacks of the row projections. Run once per step, before
 * the other calls; the GEMM calls below also take the adapters they extend
 * the reduction with (the same tensors, unchanged in between). */
moe_status moe_lora_prepare(moe_shape s, int32_t r, float scale, const void* a_gate, const void* b_gate,
                            const void* a_up, const void* b_up, const void* a_down, const void* b_down, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* moe_gemm_gate_up with the adapters: Z = x_perm [sA_gate; sA_up]^T [T*k,2rp]
 * into ws, then G, U, A over the extended reduction, whose B side is
 * b_gate [E,I,r] for the gate columns and b_up for the up columns. */
moe_status moe_lora_gemm_gate_up(moe_shape s, int32_t r, const void* x_perm, const int32_t* offsets,
                                 const void* w_gate, const void* w_up, const void* b_gate, const void* b_up, void* g,
                                 void* u, void* a, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_gemm_down with the adapters: Z_down = a (sA_down)^T into ws, then
 * o_perm over the extended reduction (B side b_down [E,H,r]). */
moe_status moe_lora_gemm_down(moe_shape s, int32_t r, const void* a, const int32_t* offsets, const void* w_down,
                              const void* b_down, void* o_perm, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_gemm_down_dgrad with the adapters: Y_down = do_perm sB_down into ws,
 * then dA over the extended reduction (its k-rows: a_down [E,r,I]) and the
 * SwiGLU backward into dgu. */
moe_status moe_lora_gemm_down_dgrad(moe_shape s, int32_t r, const void* do_perm, const int32_t* offsets,
                                    const void* w_down, const void* a_down, const void* g, const void* u, void* dgu,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_gemm_gate_up_dgrad with the adapters: Y_gu = [dG sB_gate | dU sB_up]
 * into ws, then dx_perm over the extended reduction (its k-rows: a_gate,
 * then a_up, [E,r,H]). */
moe_status moe_lora_gemm_gate_up_dgrad(moe_shape s, int32_t r, const void* dgu, const int32_t* offsets,
                                       const void* w_gate, const void* w_up, const void* a_gate, const void* a_up,
                                       void* dx_perm, void* ws, size_t ws_bytes, hipStream_t stream);

/* Without x_perm and do_perm (the gathered chain: moe_permute_fused, then
 * moe_combine_bwd with do_perm NULL): moe_lora_gemm_gate_up reading x [T,H]
 * through row_token (Z from x's rows likewise), and moe_lora_gemm_down_dgrad
 * reading dy [T,H] through row_token with the routing weight row_weight[p]
 * applied in fp32 to the whole sum (the extension included) before the
 * SwiGLU backward, as moe_gemm_down_dgrad_dy. moe_lora_gemm_down and
 * moe_lora_gemm_gate_up_dgrad are the same calls in both chains. */
moe_status moe_lora_gemm_gate_up_gathered(moe_shape s, int32_t r, const void* x, const int32_t* row_token,
                                          const int32_t* offsets, const void* w_gate, const void* w_up,
                                          const void* b_gate, const void* b_up, void* g, void* u, void* a, void* ws,
                                          size_t ws_bytes, hipStream_t stream);
moe_status moe_lora_gemm_down_dgrad_dy(moe_shape s, int32_t r, const void* dy, const int32_t* row_token,
                                       const float* row_weight, const int32_t* offsets, const void* w_down,
                                       const void* a_down, const void* g, const void* u, void* dgu, void* ws,
                                       size_t ws_bytes, hipStream_t stream);

/* The adapter gradients of the gathered unmerged chain, as
 * moe_lora_grads_gathered: the two projections that carry dO = w dy again
 * with the weight, then the outer products reading x and dy through
 * row_token. */
moe_status moe_lora_grads_unmerged_gathered(moe_shape s, int32_t r, const void* x, const int32_t* row_token,
                                            const float* row_weight, const void* act, const void* dgu, const void* dy,
                                            const int32_t* offsets, float* da_gate, float* db_gate, float* da_up,
                                            float* db_up, float* da_down, float* db_down, void* ws, size_t ws_bytes,
                                            hipStream_t stream);

/* The six adapter gradients (as moe_lora_grads) from the projections the
 * four calls above left in ws: the outer products only. */
moe_status moe_lora_grads_unmerged(moe_shape s, int32_t r, const void* x_perm, const void* act, const void* dgu,
                                   const void* do_perm, const int32_t* offsets, float* da_gate, float* db_gate,
                                   float* da_up, float* db_up, float* da_down, float* db_down, void* ws,
                                   size_t ws_bytes, hipStream_t stream);

/* fp8 activations x MXFP4 weights for the inference forward: the 4-bit
 * expert weights of the sourcepulse summary ("Quick Start & Requirements":
 * bitsandbytes 4-bit; "Limitations & Caveats": the fused 4-bit
 * dequantisation), in the microscaling FP4 format gfx950's matrix cores
 * multiply natively against E4M3 operands. Weight elements as in
 * moe_quantize_mxfp4_rows (E2M1, one E8M0 scale per 32 along K); the
 * activations stay E4M3 with one scale per row (moe_quantize_fp8_rows). The
 * matrix core applies both scales, so each product is exactly
 * dequant(a) * dequant(w), summed in fp32.
 *
 * moe_quantize_mxfp4_weights: a stacked weight w [E,N,K] bf16 (w_gate,
 * w_up [E,I,H]; w_down [E,H,I]) -> codes q [E,N,K/2] and scales e8
 * stored block-major per expert, [E,K/32,N] (the byte for expert e, block b
 * of row n at (e * K/32 + b) * N + n), the layout the GEMMs below read.
 * Codes and scales equal those of moe_quantize_mxfp4_rows on the E*N rows.
 * K % 32 == 0 (MOE_EINVAL otherwise); E*N < 2^31 (MOE_EUNSUPPORTED). */
moe_status moe_quantize_mxfp4_weights(int32_t E, int32_t N, int32_t K, const void* w, uint8_t* q, uint8_t* e8,
                                      hipStream_t stream);

/* moe_gemm_gate_up_fp8 with MXFP4 weights: wq_gate, wq_up [E,I,H/2] codes,
 * w_gate_e8, w_up_e8 [E,H/32,I] scales (moe_quantize_mxfp4_weights); the
 * rest (xq, x_e8, a, the SwiGLU epilogue) and the shape limits as there. */
moe_status moe_gemm_gate_up_mxfp4(moe_shape s, const uint8_t* xq, const uint8_t* x_e8, const int32_t* row_token,
                                  const int32_t* offsets, const uint8_t* wq_gate, const uint8_t* w_gate_e8,
                                  const uint8_t* wq_up, const uint8_t* w_up_e8, void* a, hipStream_t stream);

/* moe_gemm_down_fp8 with MXFP4 weights: wq_down [E,H,I/2] codes, w_down_e8
 * [E,I/32,H] scales; the rest as there. */
moe_status moe_gemm_down_mxfp4(moe_shape s, const uint8_t* aq, const uint8_t* a_e8, const int32_t* offsets,
                               const uint8_t* wq_down, const uint8_t* w_down_e8, const float* row_weight,
                               void* o_perm, hipStream_t stream);

/* moe_forward_fused_fp8 with the two MXFP4 GEMMs above in place of the fp8
 * ones: the same arguments, buffers, workspace and errors, the weights as
 * moe_quantize_mxfp4_weights writes them. */
moe_status moe_forward_fused_mxfp4(moe_shape s, const void* x, const void* w_router, const float* logit_bias,
                                   const uint8_t* wq_gate, const uint8_t* w_gate_e8, const uint8_t* wq_up,
                                   const uint8_t* w_up_e8, const uint8_t* wq_down, const uint8_t* w_down_e8,
                                   float* logits, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                                   int32_t* sorted_to_flat, int32_t* flat_to_sorted, int32_t* row_token,
                                   float* row_weight, uint8_t* xq, uint8_t* x_e8, void* a, uint8_t* aq, uint8_t* a_e8,
                                   void* o_perm, void* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of device workspace for moe_lora_grads at this shape and rank (0 if
 * either is rejected): the scaled adapters and the rank-wide row
 * projections. */
size_t moe_lora_workspace_bytes(moe_shape s, int32_t r);

/* Adapter gradients of the stage on the merged weights (chain rule through
 * W' = W + s B A: dA = s B^T dW', dB = s dW' A^T, with dW' the plain weight
 * gradient, formed here without dW'): over each expert's sorted rows,
 *   dB_gate = s dG^T (x_perm A_gate^T)   dA_gate = s (dG B_gate)^T x_perm
 *   dB_up   = s dU^T (x_perm A_up^T)     dA_up   = s (dU B_up)^T x_perm
 *   dB_down = s do_perm^T (a A_down^T)   dA_down = s (do_perm B_down)^T a
 * Inputs (bf16, from the forward and backward on W'): x_perm [T*k,H], a (the
 * activations) [T*k,I], dgu = [dG | dU] [T*k,2I] (moe_gemm_down_dgrad),
 * do_perm [T*k,H], offsets [E+1], the adapters. Outputs: fp32 da_* [E,r,K]
 * and db_* [E,N,r], overwritten; an expert with no rows gets zeros. The
 * scaled adapters and the projections x_perm (sA)^T, dY (sB) are rounded to
 * bf16 once; every sum is fp32. Requires shape.dtype MOE_BF16; ws of
 * ws_bytes >= moe_lora_workspace_bytes(s, r), else MOE_EWORKSPACE;
 * T k max(H, 2I) < 2^30 (32-bit byte offsets of the sorted rows), else
 * MOE_EUNSUPPORTED. */
moe_status moe_lora_grads(moe_shape s, int32_t r, float scale, const void* x_perm, const void* act, const void* dgu,
                          const void* do_perm, const int32_t* offsets, const void* a_gate, const void* b_gate,
                          const void* a_up, const void* b_up, const void* a_down, const void* b_down, float* da_gate,
                          float* db_gate, float* da_up, float* db_up, float* da_down, float* db_down, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* The same adapter gradients without x_perm and do_perm (unsloth PR #3812:
 * the grouped GEMMs read rows through the gather indices; the routing weight
 * applied inside the expert computation): row p of x_perm is row
 * row_token[p] of x [T,H], and row p of do_perm is row_weight[p] *
 * dy[row_token[p]] (dy [T,H] bf16, the stage's upstream gradient;
 * row_token, row_weight [T*k] from moe_permute_fused). The weight is applied
 * in fp32 to the two rank-wide projections that carry dO (a A_down^T for
 * dB_down, dy B_down for dA_down) before their rounding to bf16, so results
 * are within rounding of moe_lora_grads, not bit-identical. Training chain
 * without x_perm and do_perm: moe_permute_fused -> moe_gemm_gate_up_gathered
 * -> moe_gemm_down -> moe_combine; moe_combine_bwd (do_perm NULL) ->
 * moe_gemm_down_dgrad_dy -> moe_gemm_gate_up_dgrad -> this ->
 * moe_unpermute_sum -> moe_route_bwd. Same limits and errors as
 * moe_lora_grads; every pointer non-NULL (MOE_EINVAL). */
moe_status moe_lora_grads_gathered(moe_shape s, int32_t r, float scale, const void* x, const int32_t* row_token,
                                   const float* row_weight, const void* act, const void* dgu, const void* dy,
                                   const int32_t* offsets, const void* a_gate, const void* b_gate, const void* a_up,
                                   const void* b_up, const void* a_down, const void* b_down, float* da_gate,
                                   float* db_gate, float* da_up, float* db_up, float* da_down, float* db_down,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Down data gradient without do_perm (the data-gradient half of
 * moe_gemm_down_bwd_dy, for callers that train no frozen W_down, such as
 * the adapter step): dA[p] = row_weight[p] (dy[row_token[p]] W_down[e]) in
 * fp32, then the SwiGLU backward with the saved g, u into dgu = [dG | dU]
 * [T*k, 2I] (bf16). bf16 only and T*H*2 < 2^31 (MOE_EUNSUPPORTED otherwise);
 * every pointer non-NULL (MOE_EINVAL). */
moe_status moe_gemm_down_dgrad_dy(moe_shape s, const void* dy, const int32_t* row_token, const float* row_weight,
                                  const int32_t* offsets, const void* w_down, const void* g, const void* u, void* dgu,
                                  hipStream_t stream);

/* A static, human-readable name for a status code. */
const char* moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
