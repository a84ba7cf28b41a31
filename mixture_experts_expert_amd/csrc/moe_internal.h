// Internal declarations shared by the HIP sources of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

// ---------------------------------------------------------------------------
// Element types. bf16 travels as raw uint16 bit patterns.
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Round to nearest, ties to even; NaN stays NaN. gfx950 converts in one
// instruction (v_cvt_pk_bf16_f32), two values at a time.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f)); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <class T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static float to_f32(float v) { return v; }
  __device__ __forceinline__ static float from_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ __forceinline__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

__device__ __forceinline__ float sigmoidf_dev(float g) { return 1.0f / (1.0f + expf(-g)); }

// Wave-wide sum (butterfly over the 64 lanes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Permute workspace layout (bytes from the start of ws).
// ---------------------------------------------------------------------------
constexpr int kPermBlock = 1024;  // (token, slot) entries per indexing block

struct WsLayout {
  size_t hist_off;   // int32 [nblocks][E] per-block counts, then per-block bases
  size_t hist_bytes;
  size_t dgu_off;    // dtype [T*k][2I]: dG | dU for the backward
  size_t dgu_bytes;
  size_t part_off;   // fp32 [part_tiles][256][256]: split-K partial weight-gradient tiles
  size_t part_bytes;
  size_t total;
};

// Workgroups of a grouped-GEMM launch (one per CU, a multiple of 8) on the
// current device, and the most partial tiles a weight-gradient launch of
// shape s can leave for its reduction (bf16 only; 0 for fp32).
int gemm_grid();
int64_t wgrad_part_tiles(const moe_shape& s);

WsLayout ws_layout(const moe_shape& s);

// ---------------------------------------------------------------------------
// Launchers (each returns hipGetLastError() after enqueueing).
// ---------------------------------------------------------------------------
hipError_t launch_route(const moe_shape& s, const void* x, const void* wr, const float* bias, float* logits,
                        int32_t* idx, float* w, hipStream_t st);
hipError_t launch_route_bwd(const moe_shape& s, const float* gw, const float* w, const int32_t* idx,
                            float* d_logits, hipStream_t st);
hipError_t launch_permute(const moe_shape& s, const int32_t* idx, const void* x, int32_t* counts,
                          int32_t* offsets, int32_t* s2f, int32_t* f2s, void* x_perm, void* ws,
                          hipStream_t st);
hipError_t launch_combine(const moe_shape& s, const void* o_perm, const float* w, const int32_t* f2s, void* y,
                          hipStream_t st);
hipError_t launch_combine_bwd(const moe_shape& s, const void* dy, const void* o_perm, const float* w,
                              const int32_t* f2s, void* do_perm, float* gw, hipStream_t st);
hipError_t launch_permute_rows(const moe_shape& s, const int32_t* idx, const float* w, const void* x,
                               int32_t* counts, int32_t* offsets, int32_t* s2f, int32_t* f2s, int32_t* row_token,
                               float* row_weight, void* x_perm, void* ws, hipStream_t st);
hipError_t launch_permute_fused(const moe_shape& s, const int32_t* idx, const float* w, int32_t* counts,
                                int32_t* offsets, int32_t* s2f, int32_t* f2s, int32_t* row_token, float* row_weight,
                                void* ws, hipStream_t st);
// The allocation-free sort: the per-block histograms in the library's static
// scratch (kScratchBytes per device) instead of a workspace; the caller checks
// sort_hist_bytes(s) <= kScratchBytes first.
constexpr size_t kScratchBytes = 4u << 20;
size_t sort_hist_bytes(const moe_shape& s);
hipError_t launch_permute_fused_noalloc(const moe_shape& s, const int32_t* idx, const float* w, int32_t* counts,
                                        int32_t* offsets, int32_t* s2f, int32_t* f2s, int32_t* row_token,
                                        float* row_weight, hipStream_t st);
hipError_t launch_unpermute_sum(const moe_shape& s, const void* dx_perm, const int32_t* f2s, void* dx,
                                hipStream_t st);

// The six grouped GEMMs of the stage. Operand roles per mode (all row-major,
// rows sorted by expert; dgu is [T*k, 2I] with dG in columns [0, I) and dU in
// [I, 2I)):
//   GEMM_GATEUP        a = x_perm,  b0 = w_gate, b1 = w_up  -> out0 = g, out1 = u, out2 = a
//   GEMM_DOWN          a = act,     b0 = w_down             -> out0 = o_perm
//   GEMM_DGRAD_DOWN    a = do_perm, b0 = w_down, g_in, u_in -> out0 = dgu
//   GEMM_DGRAD_GATEUP  a = dgu,     b0 = w_gate, b1 = w_up  -> out0 = dx_perm
//   GEMM_WGRAD_DOWN    a = do_perm, b0 = act                -> dw0 = dw_down
//   GEMM_WGRAD_GATEUP  a = dgu,     b0 = x_perm             -> dw0 = dw_gate, dw1 = dw_up
enum GemmMode : int {
  GEMM_GATEUP = 0,
  GEMM_DOWN = 1,
  GEMM_DGRAD_DOWN = 2,
  GEMM_DGRAD_GATEUP = 3,
  GEMM_WGRAD_DOWN = 4,
  GEMM_WGRAD_GATEUP = 5
};

struct GemmArgs {
  const int32_t* offsets;
  float* part;  // weight gradients: split-K partial tiles (workspace)
  const void* a;
  const void* b0;
  const void* b1;
  const void* g_in;
  const void* u_in;
  void* out0;
  void* out1;
  void* out2;
  void* out3;   // GATEUP: a_w = bf16(row_weight[p] a[p]) (with row_weight)
  float* dw0;
  float* dw1;
  int accumulate;
  const int32_t* row_token;  // GATEUP: row p of A, WGRAD_GATEUP: k-row p of B is row row_token[p] of x [T][H];
                             // DGRAD_DOWN: row p of A, WGRAD_DOWN: k-row p of A is row row_token[p] of dy [T][H]
  const float* row_weight;   // DOWN: output row p scaled by row_weight[p]; DGRAD_DOWN with row_token: dA row p
                             // scaled by it; GATEUP with out3: a_w row p
  // fp8 GATEUP (with row_token) and DOWN (with row_weight): a and b* hold
  // E4M3 codes; E8M0 scales per sorted row of a and per weight row.
  const uint8_t* a_scale;
  const uint8_t* b0_scale;
  const uint8_t* b1_scale;
  // With a_scale: b0/b1 hold MXFP4 weights instead (E2M1 codes [E][N][K/2],
  // even k in the low nibble) and b*_scale their E8M0 block scales stored
  // block-major, [E][K/32][N].
  int b_fp4;
  // Extended reduction (bf16 GATEUP, DOWN, DGRAD_DOWN, DGRAD_GATEUP over
  // sorted rows): kx > 0 (a multiple of 32) more k past the main K, A's
  // from ax [T*k][kx], B's from rank-kxr adapters padded with zeros to kxp
  // (kx = kxp, or 2 kxp for gate/up: the gate half, then the up half):
  // bx0 (gate or down) and bx1 (up), [E][N][kxr] for GATEUP and DOWN,
  // [E][kxr][N] for the data gradients.
  const void* ax;
  const void* bx0;
  const void* bx1;
  int kx, kxr, kxp;
};

hipError_t launch_gemm_bf16(GemmMode mode, const moe_shape& s, const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_f32(GemmMode mode, const moe_shape& s, const GemmArgs& a, hipStream_t st);

inline hipError_t launch_gemm(GemmMode mode, const moe_shape& s, const GemmArgs& a, hipStream_t st) {
  return s.dtype == MOE_BF16 ? launch_gemm_bf16(mode, s, a, st) : launch_gemm_f32(mode, s, a, st);
}
// Rows [rows][K] of bf16 (K % 32 == 0) -> MXFP4: codes q [rows][K/2] (two
// per byte, the even element in the low nibble) and one E8M0 scale per 32
// elements, e8 [rows][K/32] (mxfp4.hip); with kmajor_rows = R > 0 the rows
// come in groups of R (one expert's weight) and the scales of a group are
// stored block-major, [K/32][R].
hipError_t launch_quantize_mxfp4_rows(int rows, int K, const void* in, uint8_t* q, uint8_t* e8, int kmajor_rows,
                                      hipStream_t st);
// Rows [rows, K] of bf16 -> OCP E4M3 codes with a power-of-two scale per row
// (E8M0 byte). K % 8 == 0. e8 has one byte per row, or, with flat_to_sorted
// (a [rows * k] map), one per sorted row: the scale of row r lands at
// flat_to_sorted[r k + j] for every j < k.
hipError_t launch_quantize_fp8_rows(int rows, int K, const void* in, uint8_t* q, uint8_t* e8,
                                    const int32_t* flat_to_sorted, int k, hipStream_t st);

// A data gradient and a weight gradient that read the same inputs, in one
// launch for bf16 (DGRAD_DOWN with WGRAD_DOWN, DGRAD_GATEUP with
// WGRAD_GATEUP); f32 runs them one after the other.
hipError_t launch_gemm_pair_bf16(GemmMode ma, GemmMode mb, const moe_shape& s, const GemmArgs& ga, const GemmArgs& gb,
                                 hipStream_t st);
inline hipError_t launch_gemm_pair(GemmMode ma, GemmMode mb, const moe_shape& s, const GemmArgs& ga,
                                   const GemmArgs& gb, hipStream_t st) {
  if (s.dtype == MOE_BF16) return launch_gemm_pair_bf16(ma, mb, s, ga, gb, st);
  const hipError_t err = launch_gemm_f32(ma, s, ga, st);
  return err != hipSuccess ? err : launch_gemm_f32(mb, s, gb, st);
}


// Low-rank adapters (lora.hip). The projections pad the rank to rp = 32, 64
// or 128 (the padding rows of the scaled adapters are zeros).
int lora_padded_rank(int r);

struct LoraLayout {  // byte offsets in the adapter-gradient workspace
  size_t sa_gu, sa_d, sbt_gu, sbt_d;  // bf16 scaled adapter stacks
  size_t z_gu, z_d, y_gu, y_d;        // bf16 row projections [T*k][2rp | rp]
  size_t plan;                        // split plan of the outer products (descriptors)
  size_t part;                        // fp32 partial tiles of split outer products
  size_t total;
};
LoraLayout lora_layout(const moe_shape& s, int r);

struct LoraArgs {
  const int32_t* offsets;
  const void* x_perm;   // [T*k][H], or x [T][H] with row_token
  const void* act;      // [T*k][I]
  const void* dgu;      // [T*k][2I]
  const void* do_perm;  // [T*k][H], or dy [T][H] with row_token (dO row p = row_weight[p] dy[row_token[p]])
  const int32_t* row_token;  // optional: x_perm and do_perm are x and dy read through it
  const float* row_weight;
  const void *a_gate, *b_gate, *a_up, *b_up, *a_down, *b_down;
  float *da_gate, *db_gate, *da_up, *db_up, *da_down, *db_down;
};

hipError_t launch_lora_merge(int E, int N, int K, int r, float s, const void* w, const void* a, const void* b,
                             void* w_out, hipStream_t st);
// The same with the frozen W as E4M3 codes wq [E][N][K] and E8M0 row scales
// w8 [E][N]: W' = bf16(deq(wq) + s B A).
hipError_t launch_lora_merge_fp8(int E, int N, int K, int r, float s, const uint8_t* wq, const uint8_t* w8,
                                 const void* a, const void* b, void* w_out, hipStream_t st);
// The same over MXFP4 codes wq [E][N][K/2] with E8M0 scales w8 [E][N][K/32]:
// W' = bf16(deq(wq) + s B A).
hipError_t launch_lora_merge_mxfp4(int E, int N, int K, int r, float s, const uint8_t* wq, const uint8_t* w8,
                                   const void* a, const void* b, void* w_out, hipStream_t st);
hipError_t launch_lora_grads(const moe_shape& s, int r, float scale, const LoraArgs& g, void* ws, hipStream_t st);
// The unmerged adapter step (lora.hip): the scaled stacks of the row
// projections from the adapters in g (launch_lora_prepare, once per step;
// the GEMMs' K extensions read the adapters themselves); one row projection
// (launch_lora_project: 0 Z_gu = x_perm sA_gu^T, 1 Y_gu = dgu sB_gu, 2 Z_d =
// act sA_d^T, 3 Y_d = do_perm sB_d; with tok, the rows are those of x or dy
// [T][K] read through it, and with rw, output row p is scaled by rw[p] in
// fp32) into the workspace; the adapter gradients from the projections held
// there (launch_lora_outer).
hipError_t launch_lora_prepare(const moe_shape& s, int r, float scale, const LoraArgs& g, void* ws, hipStream_t st);
hipError_t launch_lora_project(const moe_shape& s, int r, int which, const void* in, const int32_t* offsets,
                               void* ws, hipStream_t st, const int32_t* tok = nullptr, const float* rw = nullptr);
hipError_t launch_lora_outer(const moe_shape& s, int r, const LoraArgs& g, void* ws, hipStream_t st);

}  // namespace moe
