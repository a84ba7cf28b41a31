// Low-rank adapters on the frozen experts (unsloth PR #3812, the LoRA path
// of the grouped GEMM; axolotl issue #3155, fine-tuning Qwen3 MoE).
//
// Forward and data gradients run the plain stage on merged weights
// W' = W + s B A (one pass over each projection, merge_kernel below). The
// adapter gradients
//   dB = s dY^T (X A^T),   dA = s (dY B)^T X
// (dY, X per projection: dG or dU with the sorted hidden states, dO with the
// expert activations) are low-rank grouped GEMMs, run on the grouped-GEMM
// kernels with their shapes read differently: the row projections X (sA)^T
// and dY (sB) as "down" GEMMs (reduction over the row length, output width
// the padded rank), and the outer products as "down weight gradients" over
// each expert's rows. The frozen weights get no gradient.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kMT = 128;          // merge tile: 128 weight rows x 128 weight columns of one expert
constexpr int kMaxRank = 128;
constexpr int kLdsRow = kMaxRank + 8;  // A^T row in LDS (bf16); +8 keeps rows 16-byte aligned and off one bank

__device__ __forceinline__ float bf16f(bf16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

// W'[e][n][c] = bf16(W[e][n][c] + s * sum_j B[e][n][j] A[e][j][c]): the sum
// on the matrix cores (v_mfma_f32_32x32x16_bf16, exact bf16 products, fp32
// accumulation), the scale and the add in fp32, one rounding.
//
// Block: 128 columns x 128 rows of expert blockIdx.z, 4 wavefronts of
// 64 x 64 (2 x 2 MFMA blocks of 32 x 32). MFMA rows are weight columns
// (operand: A^T, staged transposed in LDS), MFMA columns weight rows
// (operand: B's rows, 16 contiguous bytes per lane straight from memory).
// Lane l then holds, per block and i < 4, four consecutive weight columns
// 8i + 4(l/32) .. + 3 of weight row l%32; a half-wave exchange pairs them
// into eight (16 bytes) so W is read and W' written in 16-byte pieces. The
// W loads are issued before the reduction so that they are in flight during it.
// w_out may be w: every element is read and written by the same lane.
__global__ __launch_bounds__(kThreads) void merge_kernel(int N, int K, int r, float s, const bf16_t* __restrict__ w,
                                                         const bf16_t* __restrict__ a, const bf16_t* __restrict__ b,
                                                         bf16_t* w_out) {
  __shared__ __attribute__((aligned(16))) bf16_t at[kMT * kLdsRow];
  const int e = blockIdx.z;
  const int c0 = blockIdx.x * kMT, n0 = blockIdx.y * kMT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wc = wave & 1, wn = wave >> 1;
  const int h = lane >> 5, l32 = lane & 31;
  const int r16 = (r + 15) & ~15;
  const int64_t wbase = static_cast<int64_t>(e) * N * K;

  // This lane's W pieces: block (tc, tn), pair p -> row n, columns col .. col + 7.
  uint4 wv[2][2][2];
#pragma unroll
  for (int tc = 0; tc < 2; ++tc)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int n = n0 + wn * 64 + tn * 32 + l32;
        const int col = c0 + wc * 64 + tc * 32 + 16 * p + 8 * h;
        wv[tc][tn][p] = n < N && col < K ? *reinterpret_cast<const uint4*>(w + wbase + static_cast<int64_t>(n) * K + col)
                                         : make_uint4(0, 0, 0, 0);
      }

  // A[e][j][c0 .. c0 + 127] -> at[c][j] (zeros past r and past K).
  const bf16_t* ae = a + static_cast<int64_t>(e) * r * K;
  for (int q = tid; q < r16 * (kMT / 8); q += kThreads) {
    const int j = q / (kMT / 8), ch = q % (kMT / 8);
    const int col = c0 + ch * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < r && col < K) v = *reinterpret_cast<const uint4*>(ae + static_cast<int64_t>(j) * K + col);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 8; ++t) at[(ch * 8 + t) * kLdsRow + j] = static_cast<bf16_t>(u[t >> 1] >> (16 * (t & 1)));
  }
  __syncthreads();

  f32x16 acc[2][2];
#pragma unroll
  for (int tc = 0; tc < 2; ++tc)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) acc[tc][tn] = f32x16{};
  const bf16_t* be = b + static_cast<int64_t>(e) * N * r;
  for (int j0 = 0; j0 < r16; j0 += 16) {
    const int j = j0 + 8 * h;  // this lane's 8 reduction indices
    bf16x8 fa[2], fb[2];
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
      fa[tc] = *reinterpret_cast<const bf16x8*>(&at[(wc * 64 + tc * 32 + l32) * kLdsRow + j]);
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      const int n = n0 + wn * 64 + tn * 32 + l32;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < N && j < r) v = *reinterpret_cast<const uint4*>(be + static_cast<int64_t>(n) * r + j);
      fb[tn] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
        acc[tc][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tc], fb[tn], acc[tc][tn], 0, 0, 0);
  }

#pragma unroll
  for (int tc = 0; tc < 2; ++tc)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        // Columns 16p .. 16p + 15 of the block: lane half 0 keeps 16p + 0..3
        // and takes 16p + 4..7 from its partner; half 1 takes 16p + 8..11 and
        // keeps 16p + 12..15.
        float v[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float mine0 = acc[tc][tn][4 * (2 * p) + q], mine1 = acc[tc][tn][4 * (2 * p + 1) + q];
          const float other = __shfl_xor(h ? mine0 : mine1, 32, 64);
          v[q] = h ? other : mine0;
          v[4 + q] = h ? mine1 : other;
        }
        const int n = n0 + wn * 64 + tn * 32 + l32;
        const int col = c0 + wc * 64 + tc * 32 + 16 * p + 8 * h;
        if (n >= N || col >= K) continue;
        const uint4 wi = wv[tc][tn][p];
        const uint32_t win[4] = {wi.x, wi.y, wi.z, wi.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = __uint_as_float(win[q] << 16) + s * v[2 * q];
          const float hi = __uint_as_float(win[q] & 0xffff0000u) + s * v[2 * q + 1];
          o[q] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
        }
        *reinterpret_cast<uint4*>(w_out + wbase + static_cast<int64_t>(n) * K + col) = make_uint4(o[0], o[1], o[2], o[3]);
      }
}

// Stacked, scaled adapter rows, each block padded to rp rows:
//   out[e][blk rp + j][c] = bf16(s in_blk[e][j][c]) for j < r, else 0,
// blk < 2 when in1 is given (gate then up), else blk = 0; in_blk [E][r][K].
__global__ __launch_bounds__(kThreads) void stack_a_kernel(int E, int r, int rp, int K, float s,
                                                           const bf16_t* __restrict__ in0,
                                                           const bf16_t* __restrict__ in1, bf16_t* __restrict__ out) {
  const int nb = in1 ? 2 : 1;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t per = static_cast<int64_t>(nb) * rp * K;
  if (q >= per * E) return;
  const int e = static_cast<int>(q / per);
  const int64_t rem = q - e * per;
  const int row = static_cast<int>(rem / K), c = static_cast<int>(rem - static_cast<int64_t>(row) * K);
  const int blk = row / rp, j = row - blk * rp;
  float v = 0.0f;
  if (j < r) v = s * bf16f((blk ? in1 : in0)[(static_cast<int64_t>(e) * r + j) * K + c]);
  out[q] = f32_to_bf16(v);
}

// Block-diagonal transposed stack: out[e][J][c], J < nb rp, c < nb C, with
// J = bj rp + j, c = bc C + cc: bf16(s in_bj[e][cc][j]) where bj == bc and
// j < r, else 0; in_b [E][C][r], nb = 2 when in1 is given.
__global__ __launch_bounds__(kThreads) void blockdiag_t_kernel(int E, int C, int r, int rp, float s,
                                                               const bf16_t* __restrict__ in0,
                                                               const bf16_t* __restrict__ in1,
                                                               bf16_t* __restrict__ out) {
  const int nb = in1 ? 2 : 1;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t per = static_cast<int64_t>(nb) * rp * nb * C;
  if (q >= per * E) return;
  const int e = static_cast<int>(q / per);
  const int64_t rem = q - e * per;
  const int J = static_cast<int>(rem / (nb * C)), c = static_cast<int>(rem - static_cast<int64_t>(J) * nb * C);
  const int bj = J / rp, j = J - bj * rp, bc = c / C, cc = c - bc * C;
  float v = 0.0f;
  if (bj == bc && j < r) v = s * bf16f((bj ? in1 : in0)[(static_cast<int64_t>(e) * C + cc) * r + j]);
  out[q] = f32_to_bf16(v);
}

// dst[e][i][j] = src[e][row0 + i][col0 + j] for i < rows, j < cols; src has
// src_rows rows of src_cols floats per expert.
__global__ __launch_bounds__(kThreads) void extract_kernel(int E, int rows, int cols, const float* __restrict__ src,
                                                           int src_rows, int src_cols, int row0, int col0,
                                                           float* __restrict__ dst) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t per = static_cast<int64_t>(rows) * cols;
  if (q >= per * E) return;
  const int e = static_cast<int>(q / per);
  const int64_t rem = q - e * per;
  const int i = static_cast<int>(rem / cols), j = static_cast<int>(rem - static_cast<int64_t>(i) * cols);
  dst[q] = src[(static_cast<int64_t>(e) * src_rows + row0 + i) * src_cols + col0 + j];
}

inline unsigned blocks_for(int64_t n) { return static_cast<unsigned>(ceil_div64(n, kThreads)); }

// out [M, N] = rows [M, K] x W[e]^T over each expert's rows, W [E, N, K]: the
// "down" GEMM with H = N, I = K.
hipError_t row_projection(const moe_shape& s, int N, int K, const int32_t* offsets, const void* rows, const void* w,
                          void* out, hipStream_t st) {
  GemmArgs g{};
  g.offsets = offsets;
  g.a = rows;
  g.b0 = w;
  g.out0 = out;
  return launch_gemm(GEMM_DOWN, lora_gemm_shape(s, N, K), g, st);
}

// dW [E, Mo, No] = L_e^T R_e over each expert's rows, L [M, Mo], R [M, No]:
// the "down weight gradient" GEMM with H = Mo, I = No.
hipError_t outer_product(const moe_shape& s, int Mo, int No, const int32_t* offsets, const void* L, const void* R,
                         float* dw, float* part, hipStream_t st) {
  GemmArgs g{};
  g.offsets = offsets;
  g.a = L;
  g.b0 = R;
  g.dw0 = dw;
  g.part = part;
  g.accumulate = 0;
  return launch_gemm(GEMM_WGRAD_DOWN, lora_gemm_shape(s, Mo, No), g, st);
}

}  // namespace

int lora_padded_rank(int r) { return (r + 63) & ~63; }

moe_shape lora_gemm_shape(const moe_shape& s, int H, int I) {
  moe_shape g = s;
  g.H = H;
  g.I = I;
  return g;
}

LoraLayout lora_layout(const moe_shape& s, int r) {
  LoraLayout l{};
  const int64_t M = static_cast<int64_t>(s.T) * s.k;
  const int64_t E = s.E, H = s.H, I = s.I, rp = lora_padded_rank(r);
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    const size_t o = off;
    off = (off + static_cast<size_t>(bytes) + 255) & ~static_cast<size_t>(255);
    return o;
  };
  l.sa_gu = take(E * 2 * rp * H * 2);
  l.sa_d = take(E * rp * I * 2);
  l.sbt_gu = take(E * 2 * rp * 2 * I * 2);
  l.sbt_d = take(E * rp * H * 2);
  l.z_gu = take(M * 2 * rp * 2);
  l.z_d = take(M * rp * 2);
  l.y_gu = take(M * 2 * rp * 2);
  l.y_d = take(M * rp * 2);
  l.da_gu = take(E * 2 * rp * H * 4);
  l.db_gu = take(E * 2 * I * 2 * rp * 4);
  l.da_d = take(E * rp * I * 4);
  l.db_d = take(E * H * rp * 4);
  l.part = take(static_cast<int64_t>(2 * gemm_grid()) * 256 * 256 * 4);
  l.total = off;
  return l;
}

hipError_t launch_lora_merge(int E, int N, int K, int r, float s, const void* w, const void* a, const void* b,
                             void* w_out, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(ceil_div(K, kMT)), static_cast<unsigned>(ceil_div(N, kMT)),
                  static_cast<unsigned>(E));
  merge_kernel<<<grid, kThreads, 0, st>>>(N, K, r, s, static_cast<const bf16_t*>(w), static_cast<const bf16_t*>(a),
                                          static_cast<const bf16_t*>(b), static_cast<bf16_t*>(w_out));
  return hipGetLastError();
}

hipError_t launch_lora_grads(const moe_shape& s, int r, float scale, const LoraArgs& g, void* ws, hipStream_t st) {
  const LoraLayout l = lora_layout(s, r);
  char* base = static_cast<char*>(ws);
  bf16_t* sa_gu = reinterpret_cast<bf16_t*>(base + l.sa_gu);
  bf16_t* sa_d = reinterpret_cast<bf16_t*>(base + l.sa_d);
  bf16_t* sbt_gu = reinterpret_cast<bf16_t*>(base + l.sbt_gu);
  bf16_t* sbt_d = reinterpret_cast<bf16_t*>(base + l.sbt_d);
  void* z_gu = base + l.z_gu;
  void* z_d = base + l.z_d;
  void* y_gu = base + l.y_gu;
  void* y_d = base + l.y_d;
  float* da_gu = reinterpret_cast<float*>(base + l.da_gu);
  float* db_gu = reinterpret_cast<float*>(base + l.db_gu);
  float* part = reinterpret_cast<float*>(base + l.part);
  const int E = s.E, H = s.H, I = s.I, rp = lora_padded_rank(r);
  // With rp == r the down-projection gradients land in place.
  float* da_d = rp == r ? g.da_down : reinterpret_cast<float*>(base + l.da_d);
  float* db_d = rp == r ? g.db_down : reinterpret_cast<float*>(base + l.db_d);
  const bf16_t* a_gate = static_cast<const bf16_t*>(g.a_gate);
  const bf16_t* a_up = static_cast<const bf16_t*>(g.a_up);
  const bf16_t* a_down = static_cast<const bf16_t*>(g.a_down);
  const bf16_t* b_gate = static_cast<const bf16_t*>(g.b_gate);
  const bf16_t* b_up = static_cast<const bf16_t*>(g.b_up);
  const bf16_t* b_down = static_cast<const bf16_t*>(g.b_down);
  hipError_t err;
#define MOE_TRY(x) \
  if ((err = (x)) != hipSuccess) return err
  // Scaled, stacked adapters (bf16, rounded once): sA_gu = [sA_gate; sA_up],
  // sA_d, the transposed block diagonal of sB_gate and sB_up, sB_down^T.
  stack_a_kernel<<<blocks_for(int64_t{E} * 2 * rp * H), kThreads, 0, st>>>(E, r, rp, H, scale, a_gate, a_up, sa_gu);
  MOE_TRY(hipGetLastError());
  stack_a_kernel<<<blocks_for(int64_t{E} * rp * I), kThreads, 0, st>>>(E, r, rp, I, scale, a_down, nullptr, sa_d);
  MOE_TRY(hipGetLastError());
  blockdiag_t_kernel<<<blocks_for(int64_t{E} * 4 * rp * I), kThreads, 0, st>>>(E, I, r, rp, scale, b_gate, b_up,
                                                                               sbt_gu);
  MOE_TRY(hipGetLastError());
  blockdiag_t_kernel<<<blocks_for(int64_t{E} * rp * H), kThreads, 0, st>>>(E, H, r, rp, scale, b_down, nullptr,
                                                                           sbt_d);
  MOE_TRY(hipGetLastError());
  // Row projections Z = X (sA)^T, Y = dY (sB).
  MOE_TRY(row_projection(s, 2 * rp, H, g.offsets, g.x_perm, sa_gu, z_gu, st));    // [Z_gate | Z_up]
  MOE_TRY(row_projection(s, rp, I, g.offsets, g.act, sa_d, z_d, st));             // Z_down
  MOE_TRY(row_projection(s, 2 * rp, 2 * I, g.offsets, g.dgu, sbt_gu, y_gu, st));  // [dG sB_gate | dU sB_up]
  MOE_TRY(row_projection(s, rp, H, g.offsets, g.do_perm, sbt_d, y_d, st));        // dO sB_down
  // Outer products over each expert's rows.
  MOE_TRY(outer_product(s, 2 * I, 2 * rp, g.offsets, g.dgu, z_gu, db_gu, part, st));  // [dG | dU]^T [Z_gate | Z_up]
  MOE_TRY(outer_product(s, 2 * rp, H, g.offsets, y_gu, g.x_perm, da_gu, part, st));   // [Y_gate | Y_up]^T X
  MOE_TRY(outer_product(s, H, rp, g.offsets, g.do_perm, z_d, db_d, part, st));       // dO^T Z_down
  MOE_TRY(outer_product(s, rp, I, g.offsets, y_d, g.act, da_d, part, st));           // Y_down^T Act
  // The adapters' own blocks.
  extract_kernel<<<blocks_for(int64_t{E} * r * H), kThreads, 0, st>>>(E, r, H, da_gu, 2 * rp, H, 0, 0, g.da_gate);
  MOE_TRY(hipGetLastError());
  extract_kernel<<<blocks_for(int64_t{E} * r * H), kThreads, 0, st>>>(E, r, H, da_gu, 2 * rp, H, rp, 0, g.da_up);
  MOE_TRY(hipGetLastError());
  extract_kernel<<<blocks_for(int64_t{E} * I * r), kThreads, 0, st>>>(E, I, r, db_gu, 2 * I, 2 * rp, 0, 0,
                                                                      g.db_gate);
  MOE_TRY(hipGetLastError());
  extract_kernel<<<blocks_for(int64_t{E} * I * r), kThreads, 0, st>>>(E, I, r, db_gu, 2 * I, 2 * rp, I, rp,
                                                                      g.db_up);
  MOE_TRY(hipGetLastError());
  if (rp != r) {
    extract_kernel<<<blocks_for(int64_t{E} * r * I), kThreads, 0, st>>>(E, r, I, da_d, rp, I, 0, 0, g.da_down);
    MOE_TRY(hipGetLastError());
    extract_kernel<<<blocks_for(int64_t{E} * H * r), kThreads, 0, st>>>(E, H, r, db_d, H, rp, 0, 0, g.db_down);
    MOE_TRY(hipGetLastError());
  }
#undef MOE_TRY
  return hipSuccess;
}

}  // namespace moe
