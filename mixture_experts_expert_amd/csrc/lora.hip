// Low-rank adapters on the frozen, stacked experts (sourcepulse summary,
// "Highlighted Details": LoRA and QLoRA on the fused experts, in the fused
// adapter format; torchtune PR #2820: LoRA support for the Qwen3 MoE port).
//
// Forward and data gradients run the plain stage on merged weights
// W' = W + s B A (one pass over each projection, merge_kernel below). The
// adapter gradients
//   dB = s dY^T (X A^T),   dA = s (dY B)^T X
// (dY, X per projection: dG or dU with the sorted hidden states, dO with the
// expert activations) are low-rank grouped GEMMs: the four rank-wide row
// projections X (sA)^T and dY (sB) in one launch of proj_kernel below, and
// the outer products over each expert's rows on the grouped weight-gradient
// kernels, with their shapes read differently. The frozen weights get no
// gradient.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer loads: a wavefront-uniform base and byte range; a lane whose
// offset falls outside the range reads zeros (no branch, so the compiler
// can count the loads in flight exactly).
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes, 0x00020000);
}
__device__ __forceinline__ uint4 load16(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr int kThreads = 256;
constexpr int kMT = 128;          // merge tile: 128 weight rows x 128 weight columns of one expert
constexpr int kMergeRowTiles = 2; // row tiles per merge block
constexpr int kMaxRank = 128;
constexpr int kLdsRow = kMaxRank + 8;  // A^T row in LDS (bf16); +8 keeps rows 16-byte aligned and off one bank
constexpr int kStageRow = kMT + 4;     // fp32 stage row: 16-byte aligned, rows 4 banks apart
static_assert(kMT * kLdsRow * 2 <= kMT * kStageRow * 4, "A^T fits in the stage region");

// Workgroup barrier for LDS hand-offs: waits for this wavefront's LDS
// traffic only (s_waitcnt lgkmcnt(0), vmcnt and expcnt unconstrained: gfx9
// encoding 0xC07F), so global loads issued ahead stay in flight; a
// __syncthreads() would wait for them too. The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float bf16f(bf16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

// W'[e][n][c] = bf16(W[e][n][c] + s * sum_j B[e][n][j] A[e][j][c]): the sum
// on the matrix cores (v_mfma_f32_32x32x16_bf16, exact bf16 products, fp32
// accumulation in j order), the scale and the add in fp32, one rounding.
//
// Block: 128 columns of expert blockIdx.z and up to kMergeRowTiles tiles of
// 128 rows; 4 wavefronts, each 64 columns x 64 rows of a tile (2 x 2 MFMA
// blocks of 32 x 32). MFMA rows are weight columns: the operand is A^T,
// staged transposed in LDS once per block and then held in registers for
// every row tile. MFMA columns are weight rows: the operand is B's rows, 16
// contiguous bytes per lane straight from memory. The sums go through LDS
// (fp32, the region A^T used) so that W is read and W' written in row runs:
// 16 lanes cover a row's 256 bytes, each lane 16 bytes (the MFMA layout
// itself gives each lane 8-byte pieces of 32 different rows, which streams
// at about half the rate). A row tile's loads (B fragments and W) are
// issued during the previous tile's epilogue. NS = ceil(r / 16) reduction
// steps. w_out may be w: every element is read and written by the same
// thread.
template <int NS>
__global__ __launch_bounds__(kThreads) void merge_kernel(int N, int K, int r, float s, const bf16_t* w,
                                                         const bf16_t* __restrict__ a, const bf16_t* __restrict__ b,
                                                         bf16_t* w_out) {
  __shared__ __attribute__((aligned(16))) float lds[kMT * kStageRow];
  bf16_t* at = reinterpret_cast<bf16_t*>(lds);  // A^T [128][kLdsRow], then the fp32 stage [128][kStageRow]
  const int e = blockIdx.z;
  const int c0 = blockIdx.x * kMT, nbeg = blockIdx.y * kMT * kMergeRowTiles;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wc = wave & 1, wn = wave >> 1;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t wbase = static_cast<int64_t>(e) * N * K;
  // Row runs of the epilogue: pass q covers tile rows 16q + tid/16, columns
  // 8 (tid%16) .. + 7.
  const int rrow = tid >> 4, rcol = (tid & 15) * 8;

  // A[e][j][c0 .. c0 + 127] -> at[c][j] (zeros past r and past K).
  const bf16_t* ae = a + static_cast<int64_t>(e) * r * K;
  for (int q = tid; q < NS * 16 * (kMT / 8); q += kThreads) {
    const int j = q / (kMT / 8), ch = q % (kMT / 8);
    const int col = c0 + ch * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < r && col < K) v = *reinterpret_cast<const uint4*>(ae + static_cast<int64_t>(j) * K + col);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 8; ++t) at[(ch * 8 + t) * kLdsRow + j] = static_cast<bf16_t>(u[t >> 1] >> (16 * (t & 1)));
  }
  __syncthreads();
  bf16x8 fa[2][NS];
#pragma unroll
  for (int tc = 0; tc < 2; ++tc)
#pragma unroll
    for (int q = 0; q < NS; ++q)
      fa[tc][q] = *reinterpret_cast<const bf16x8*>(&at[(wc * 64 + tc * 32 + l32) * kLdsRow + 16 * q + 8 * h]);

  const bf16_t* be = b + static_cast<int64_t>(e) * N * r;
  const bool cok = c0 + rcol < K;
  bf16x8 fb[2][NS];
  uint4 wv[2][kMT / 16];  // W row runs of the current and the next row tile
  const rsrc_t rw = make_rsrc(w + wbase, 2 * N * K), rb = make_rsrc(be, 2 * N * r);
  auto load_tile = [&](int nt, uint4 (&wt)[kMT / 16]) __attribute__((always_inline)) {
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      const int n = nt + wn * 64 + tn * 32 + l32;  // rows past N read zeros
#pragma unroll
      for (int q = 0; q < NS; ++q) {
        const int j = 16 * q + 8 * h;
        fb[tn][q] = __builtin_bit_cast(bf16x8, load16(rb, j < r ? 2u * static_cast<uint32_t>(n * r + j) : kOutOfRange));
      }
    }
#pragma unroll
    for (int q = 0; q < kMT / 16; ++q) {
      const int n = nt + 16 * q + rrow;
      wt[q] = load16(rw, cok ? 2u * static_cast<uint32_t>(n * K + c0 + rcol) : kOutOfRange);
    }
  };
  load_tile(nbeg, wv[0]);
#pragma unroll
  for (int t = 0; t < kMergeRowTiles; ++t) {
    const int nt = nbeg + t * kMT;
    f32x16 acc[2][2];
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) {
        acc[tc][tn] = f32x16{};
#pragma unroll
        for (int q = 0; q < NS; ++q)
          acc[tc][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tc][q], fb[tn][q], acc[tc][tn], 0, 0, 0);
      }
    // The next tile's loads fly during this tile's epilogue.
    // Rows past N read zeros and are not stored: no branch, so the
    // compiler keeps these loads in flight across the epilogue's waits.
    if (t + 1 < kMergeRowTiles) load_tile(nt + kMT, wv[(t + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();  // A^T (first tile) or the previous tile's stage has been read
    // Lane l holds, per block and i < 4, columns 8i + 4(l/32) .. + 3 of row l%32.
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<float4*>(&lds[(wn * 64 + tn * 32 + l32) * kStageRow + wc * 64 + tc * 32 + 8 * i + 4 * h]) =
              make_float4(acc[tc][tn][4 * i], acc[tc][tn][4 * i + 1], acc[tc][tn][4 * i + 2], acc[tc][tn][4 * i + 3]);
    lds_barrier();
    const uint4 (&wc_t)[kMT / 16] = wv[t & 1];
#pragma unroll
    for (int q = 0; q < kMT / 16; ++q) {
      const int n = nt + 16 * q + rrow;
      if (n >= N || !cok) continue;
      const float* sp = &lds[(16 * q + rrow) * kStageRow + rcol];
      const float4 v0 = *reinterpret_cast<const float4*>(sp), v1 = *reinterpret_cast<const float4*>(sp + 4);
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      const uint32_t win[4] = {wc_t[q].x, wc_t[q].y, wc_t[q].z, wc_t[q].w};
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float lo = __uint_as_float(win[p] << 16) + s * v[2 * p];
        const float hi = __uint_as_float(win[p] & 0xffff0000u) + s * v[2 * p + 1];
        o[p] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
      }
      *reinterpret_cast<uint4*>(w_out + wbase + static_cast<int64_t>(n) * K + c0 + rcol) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

__device__ __forceinline__ uint32_t scale_pair(uint32_t v, float s) {
  const float lo = s * __uint_as_float(v << 16), hi = s * __uint_as_float(v & 0xffff0000u);
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Stacked, scaled adapter rows, each block padded to rp rows:
//   out[e][blk rp + j][c] = bf16(s in_blk[e][j][c]) for j < r, else 0,
// blk < 2 when in1 is given (gate then up), else blk = 0; in_blk [E][r][K].
// Block x = output row, threads over its 16-byte chunks.
__global__ __launch_bounds__(kThreads) void stack_a_kernel(int r, int rp, int K, float s,
                                                           const bf16_t* __restrict__ in0,
                                                           const bf16_t* __restrict__ in1, bf16_t* __restrict__ out) {
  const int row = blockIdx.x;
  const int c = (blockIdx.y * kThreads + threadIdx.x) * 8;
  if (c >= K) return;
  const int nb = in1 ? 2 : 1;
  const int e = row / (nb * rp), rem = row - e * nb * rp, blk = rem / rp, j = rem - blk * rp;
  uint4 o = make_uint4(0, 0, 0, 0);
  if (j < r) {
    const uint4 v = *reinterpret_cast<const uint4*>((blk ? in1 : in0) + (static_cast<int64_t>(e) * r + j) * K + c);
    o = make_uint4(scale_pair(v.x, s), scale_pair(v.y, s), scale_pair(v.z, s), scale_pair(v.w, s));
  }
  *reinterpret_cast<uint4*>(out + static_cast<int64_t>(row) * K + c) = o;
}

// Block-diagonal transposed stack: out[e][J][c], J < nb rp, c < nb C, with
// J = bj rp + j, c = bc C + cc: bf16(s in_bj[e][cc][j]) where bj == bc and
// j < r, else 0; in_b [E][C][r], nb = 2 when in1 is given, C % 64 == 0.
// Block (x, e): output columns 64x .. 64x + 63, all of one block column bc;
// their 64 rows of in_bc are read whole into LDS and written out transposed.
__global__ __launch_bounds__(kThreads) void blockdiag_t_kernel(int C, int r, int rp, float s,
                                                               const bf16_t* __restrict__ in0,
                                                               const bf16_t* __restrict__ in1,
                                                               bf16_t* __restrict__ out) {
  __shared__ float tile[64][kMaxRank + 1];
  const int nb = in1 ? 2 : 1;
  const int e = blockIdx.y, c0 = blockIdx.x * 64, bc = c0 / C, cc0 = c0 - bc * C;
  const int tid = threadIdx.x;
  const bf16_t* src = (bc ? in1 : in0) + (static_cast<int64_t>(e) * C + cc0) * r;
  const int c8 = r / 8;  // 16-byte pieces per row of in_bc (r % 8 == 0)
  for (int q = tid; q < 64 * c8; q += kThreads) {
    const int row = q / c8, j0 = (q - row * c8) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(src + row * r + j0);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      tile[row][j0 + 2 * t] = s * __uint_as_float(u[t] << 16);
      tile[row][j0 + 2 * t + 1] = s * __uint_as_float(u[t] & 0xffff0000u);
    }
  }
  __syncthreads();
  // Thread: output columns 8 (tid%8) .. + 7 of rows J = tid/8, tid/8 + 32, ...
  const int cq = (tid & 7) * 8;
  bf16_t* dst = out + static_cast<int64_t>(e) * nb * rp * nb * C + c0 + cq;
  for (int J = tid >> 3; J < nb * rp; J += kThreads / 8) {
    const int bj = J / rp, j = J - bj * rp;
    const bool live = bj == bc && j < r;
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float lo = live ? tile[cq + 2 * p][j] : 0.0f, hi = live ? tile[cq + 2 * p + 1][j] : 0.0f;
      o[p] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
    }
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(J) * nb * C) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// dst[e][i][j] = src[e][row0 + i][col0 + j] for i < rows, j < cols (cols,
// col0 and src_cols multiples of 4); src has src_rows rows of src_cols
// floats per expert. One thread per 16 bytes.
__global__ __launch_bounds__(kThreads) void extract_kernel(int64_t total4, int rows, int cols, const float* __restrict__ src,
                                                           int src_rows, int src_cols, int row0, int col0,
                                                           float* __restrict__ dst) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (q >= total4) return;
  const int c4 = cols / 4;
  const int64_t row = q / c4;  // e * rows + i
  const int j = static_cast<int>(q - row * c4) * 4;
  const int64_t e = row / rows, i = row - e * rows;
  *reinterpret_cast<float4*>(dst + q * 4) =
      *reinterpret_cast<const float4*>(src + (e * src_rows + row0 + i) * src_cols + col0 + j);
}

// Rank-wide projections: out[p][n] = sum_k rows[p][k] W[e][n][k] over each
// expert e's sorted rows p, W [E][N][K], N a multiple of 64 up to 32 NB,
// K % 64 == 0; bf16 in and out, fp32 sums. One launch runs up to four such
// jobs over the same experts (the four projections of the adapter
// gradients), so that their tiles fill the chip together instead of each
// leaving a tail.
//
// Tile: 128 rows of one expert x 32 NB columns (columns past the job's N
// read zero weights and are not stored), 4 wavefronts of 32 rows. k-chunks
// of 64 go global -> registers -> LDS (double-buffered; the loads of the
// next two chunks are in flight during a chunk's MFMAs), each load
// instruction covering 8 rows x 128 bytes. MFMA rows are output columns
// (operand: W's rows), MFMA columns output rows (operand: the tile's rows),
// so a lane holds four consecutive output columns of one row; a half-wave
// exchange makes them eight for 16-byte stores. The tile list is built on
// the device from the offsets (a block-wide scan of the experts' tile
// counts), the jobs interleaved tile by tile, and cut into 8 contiguous
// ranges, one per XCD, so an expert's tiles share its W in one L2.
constexpr int kPR = 128;        // rows per projection tile
constexpr int kPK = 64;         // k-chunk
constexpr int kPLds = kPK + 8;  // LDS row (bf16): 144 bytes, rows 4 banks apart

struct ProjJob {
  const bf16_t* rows;  // [T*k][K]
  const bf16_t* w;     // [E][N][K]
  bf16_t* out;         // [T*k][N]
  int K, N;
};
struct ProjJobs {
  ProjJob job[4];
  int n;
};

template <int NB>
__global__ __launch_bounds__(kThreads) void proj_kernel(int E, const int32_t* __restrict__ offsets, ProjJobs jobs) {
  constexpr int NMAX = 32 * NB;
  __shared__ __attribute__((aligned(16))) bf16_t xs[2][kPR * kPLds];
  __shared__ __attribute__((aligned(16))) bf16_t wl[2][NMAX * kPLds];
  __shared__ int wsum[kThreads / 64];
  __shared__ int found[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;

  // Tile counts of experts 4 tid .. 4 tid + 3 and their exclusive prefix.
  int cnt[4], sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * 4 + j;
    cnt[j] = e < E ? (offsets[e + 1] - offsets[e] + kPR - 1) / kPR : 0;
    sum += cnt[j];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int start = incl - sum, per_job = 0;
#pragma unroll
  for (int v = 0; v < kThreads / 64; ++v) {
    start += v < wave ? wsum[v] : 0;
    per_job += wsum[v];
  }
  const int total = per_job * jobs.n;
  const int per_xcd = (total + 7) / 8;
  const int t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (static_cast<int>(blockIdx.x / 8) >= per_xcd || t >= total) return;  // uniform over the block
  const int jb = t % jobs.n, tt = t / jobs.n;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (tt >= start && tt < start + cnt[j]) {
      found[0] = tid * 4 + j;
      found[1] = tt - start;
    }
    start += cnt[j];
  }
  __syncthreads();
  const int e = found[0];
  const int r0 = offsets[e] + found[1] * kPR;
  const int valid = min(kPR, offsets[e + 1] - r0);
  const ProjJob& J = jobs.job[jb];
  const int K = J.K, N = J.N;
  const bf16_t* rows = J.rows;
  const bf16_t* w = J.w;
  bf16_t* out = J.out;

  // Buffer ranges start at the chunk's first column: rows past the tile's
  // valid ones fall outside and read zeros. The per-lane offsets stay fixed.
  const bf16_t* abase = rows + static_cast<int64_t>(r0) * K;
  const bf16_t* wbase = w + static_cast<int64_t>(e) * N * K;
  // 16-byte pieces of a chunk: piece q is row q / 8, bytes 16 (q % 8) of its 128.
  constexpr int PA = kPR * 8 / kThreads, PB = NMAX * 8 / kThreads;
  uint32_t oa[PA], ob[PB];
#pragma unroll
  for (int i = 0; i < PA; ++i) {
    const int q = tid + kThreads * i;
    oa[i] = 2u * static_cast<uint32_t>((q >> 3) * K) + 16u * (q & 7);
  }
#pragma unroll
  for (int i = 0; i < PB; ++i) {
    const int q = tid + kThreads * i;
    ob[i] = 2u * static_cast<uint32_t>((q >> 3) * K) + 16u * (q & 7);
  }
  uint4 pa[2][PA], pb[2][PB];  // two chunks in flight
  auto load_chunk = [&](int k0, uint4 (&qa)[PA], uint4 (&qb)[PB]) __attribute__((always_inline)) {
    // Past the last chunk the ranges are empty: the loads read zeros and
    // touch no memory, so the loop needs no branch around them.
    const bool live = k0 < K;
    const rsrc_t ra = make_rsrc(abase + (live ? k0 : 0), live ? 2 * (valid * K - k0) : 0);
    const rsrc_t rw = make_rsrc(wbase + (live ? k0 : 0), live ? 2 * (N * K - k0) : 0);
#pragma unroll
    for (int i = 0; i < PA; ++i) qa[i] = load16(ra, oa[i]);
#pragma unroll
    for (int i = 0; i < PB; ++i) qb[i] = load16(rw, ob[i]);
  };
  auto store_chunk = [&](int buf, const uint4 (&qa)[PA], const uint4 (&qb)[PB]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int q = tid + kThreads * i;
      *reinterpret_cast<uint4*>(&xs[buf][(q >> 3) * kPLds + (q & 7) * 8]) = qa[i];
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int q = tid + kThreads * i;
      *reinterpret_cast<uint4*>(&wl[buf][(q >> 3) * kPLds + (q & 7) * 8]) = qb[i];
    }
  };

  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};
  // LDS holds chunk c; register set (c + 1) % 2 holds chunk c + 1 and set
  // c % 2 takes chunk c + 2 (issued during chunk c). The chunk count is
  // rounded up to even: a chunk past the end is all zeros and adds nothing,
  // so no step, load or store needs a branch (a branch would make the
  // compiler wait for every load in flight at the join).
  const int nch = (K / kPK + 1) & ~1;
  load_chunk(0, pa[0], pb[0]);
  load_chunk(kPK, pa[1], pb[1]);
  store_chunk(0, pa[0], pb[0]);
  lds_barrier();
  auto step = [&](int c, uint4 (&na)[PA], uint4 (&nb_)[PB], uint4 (&ca)[PA], uint4 (&cb)[PB])
      __attribute__((always_inline)) {
    // na/nb_: the register set that held chunk c (free), now chunk c + 2;
    // ca/cb: chunk c + 1, stored to LDS after this chunk's MFMAs.
    const int buf = c & 1;
    load_chunk((c + 2) * kPK, na, nb_);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of this chunk's MFMAs
#pragma unroll
    for (int sl = 0; sl < kPK / 16; ++sl) {
      const bf16x8 fx = *reinterpret_cast<const bf16x8*>(&xs[buf][(wave * 32 + l32) * kPLds + 16 * sl + 8 * h]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 fw = *reinterpret_cast<const bf16x8*>(&wl[buf][(nb * 32 + l32) * kPLds + 16 * sl + 8 * h]);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw, fx, acc[nb], 0, 0, 0);
      }
    }
    store_chunk(buf ^ 1, ca, cb);
    lds_barrier();  // chunk c + 1 is in LDS; nobody reads buffer buf any more
  };
  for (int c = 0; c < nch; c += 2) {
    step(c, pa[0], pb[0], pa[1], pb[1]);
    step(c + 1, pa[1], pb[1], pa[0], pb[0]);
  }

  // Lane l: output row wave * 32 + l%32, columns 8i + 4(l/32) .. + 3 of each 32-column block.
  const int row = wave * 32 + l32;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float mine0 = acc[nb][4 * (2 * p) + q], mine1 = acc[nb][4 * (2 * p + 1) + q];
        const float other = __shfl_xor(h ? mine0 : mine1, 32, 64);
        v[q] = h ? other : mine0;
        v[4 + q] = h ? mine1 : other;
      }
      if (row >= valid || nb * 32 >= N) continue;
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = static_cast<uint32_t>(f32_to_bf16(v[2 * q])) | (static_cast<uint32_t>(f32_to_bf16(v[2 * q + 1])) << 16);
      *reinterpret_cast<uint4*>(out + static_cast<int64_t>(r0 + row) * N + nb * 32 + 16 * p + 8 * h) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// The four rank-wide projections in one launch; nmax = the widest N.
hipError_t projections(const moe_shape& s, int nmax, const int32_t* offsets, const ProjJobs& jobs, hipStream_t st) {
  const int64_t M = static_cast<int64_t>(s.T) * s.k;
  // >= the tile count (each job: at most M / 128 + E tiles), a multiple of 8.
  const unsigned grid = static_cast<unsigned>(8 * ((jobs.n * (M / kPR + s.E) + 8) / 8));
  switch (nmax / 32) {
    case 4: proj_kernel<4><<<grid, kThreads, 0, st>>>(s.E, offsets, jobs); break;
    case 8: proj_kernel<8><<<grid, kThreads, 0, st>>>(s.E, offsets, jobs); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
  l.da_g = take(E * rp * H * 4);
  l.da_u = take(E * rp * H * 4);
  l.db_gu = take(E * 2 * I * 2 * rp * 4);
  l.da_d = take(E * rp * I * 4);
  l.db_d = take(E * H * rp * 4);
  l.part = take(static_cast<int64_t>(2 * gemm_grid()) * 256 * 256 * 4);
  l.total = off;
  return l;
}

hipError_t launch_lora_merge(int E, int N, int K, int r, float s, const void* w, const void* a, const void* b,
                             void* w_out, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(ceil_div(K, kMT)), static_cast<unsigned>(ceil_div(N, kMT * kMergeRowTiles)),
                  static_cast<unsigned>(E));
  const bf16_t* wp = static_cast<const bf16_t*>(w);
  const bf16_t* ap = static_cast<const bf16_t*>(a);
  const bf16_t* bp = static_cast<const bf16_t*>(b);
  bf16_t* op = static_cast<bf16_t*>(w_out);
  switch ((r + 15) / 16) {
    case 1: merge_kernel<1><<<grid, kThreads, 0, st>>>(N, K, r, s, wp, ap, bp, op); break;
    case 2: merge_kernel<2><<<grid, kThreads, 0, st>>>(N, K, r, s, wp, ap, bp, op); break;
    case 3: merge_kernel<3><<<grid, kThreads, 0, st>>>(N, K, r, s, wp, ap, bp, op); break;
    case 4: merge_kernel<4><<<grid, kThreads, 0, st>>>(N, K, r, s, wp, ap, bp, op); break;
    case 5: merge_kernel<5><<<grid, kThreads, 0, st>>>(N, K, r, s, wp, ap, bp, op); break;
    case 6: merge_kernel<6><<<grid, kThreads, 0, st>>>(N, K, r, s, wp, ap, bp, op); break;
    case 7: merge_kernel<7><<<grid, kThreads, 0, st>>>(N, K, r, s, wp, ap, bp, op); break;
    case 8: merge_kernel<8><<<grid, kThreads, 0, st>>>(N, K, r, s, wp, ap, bp, op); break;
    default: return hipErrorInvalidValue;
  }
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
  float* db_gu = reinterpret_cast<float*>(base + l.db_gu);
  float* part = reinterpret_cast<float*>(base + l.part);
  const int E = s.E, H = s.H, I = s.I, rp = lora_padded_rank(r);
  // With rp == r the dA and dB_down gradients land in place.
  const bool padded = rp != r;
  float* da_g = padded ? reinterpret_cast<float*>(base + l.da_g) : g.da_gate;
  float* da_u = padded ? reinterpret_cast<float*>(base + l.da_u) : g.da_up;
  float* da_d = padded ? reinterpret_cast<float*>(base + l.da_d) : g.da_down;
  float* db_d = padded ? reinterpret_cast<float*>(base + l.db_d) : g.db_down;
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
  stack_a_kernel<<<dim3(E * 2 * rp, ceil_div(H / 8, kThreads)), kThreads, 0, st>>>(r, rp, H, scale, a_gate, a_up,
                                                                                     sa_gu);
  MOE_TRY(hipGetLastError());
  stack_a_kernel<<<dim3(E * rp, ceil_div(I / 8, kThreads)), kThreads, 0, st>>>(r, rp, I, scale, a_down, nullptr,
                                                                                 sa_d);
  MOE_TRY(hipGetLastError());
  blockdiag_t_kernel<<<dim3(2 * I / 64, E), kThreads, 0, st>>>(I, r, rp, scale, b_gate, b_up, sbt_gu);
  MOE_TRY(hipGetLastError());
  blockdiag_t_kernel<<<dim3(H / 64, E), kThreads, 0, st>>>(H, r, rp, scale, b_down, nullptr, sbt_d);
  MOE_TRY(hipGetLastError());
  // Row projections Z = X (sA)^T, Y = dY (sB): [Z_gate | Z_up], [dG sB_gate |
  // dU sB_up], Z_down, dO sB_down.
  {
    ProjJobs pj{};
    const bf16_t* xp = static_cast<const bf16_t*>(g.x_perm);
    pj.job[0] = {xp, sa_gu, static_cast<bf16_t*>(z_gu), H, 2 * rp};
    pj.job[1] = {static_cast<const bf16_t*>(g.dgu), sbt_gu, static_cast<bf16_t*>(y_gu), 2 * I, 2 * rp};
    pj.job[2] = {static_cast<const bf16_t*>(g.act), sa_d, static_cast<bf16_t*>(z_d), I, rp};
    pj.job[3] = {static_cast<const bf16_t*>(g.do_perm), sbt_d, static_cast<bf16_t*>(y_d), H, rp};
    pj.n = 4;
    MOE_TRY(projections(s, 2 * rp, g.offsets, pj, st));
  }
  // Outer products over each expert's rows. [Y_gate | Y_up]^T X has the
  // layout of the gate/up weight gradient with I = rp: its two halves go to
  // dA_gate and dA_up directly.
  {
    GemmArgs ga{};
    ga.offsets = g.offsets;
    ga.a = y_gu;
    ga.b0 = g.x_perm;
    ga.dw0 = da_g;
    ga.dw1 = da_u;
    ga.part = part;
    MOE_TRY(launch_gemm(GEMM_WGRAD_GATEUP, lora_gemm_shape(s, H, rp), ga, st));
  }
  MOE_TRY(outer_product(s, 2 * I, 2 * rp, g.offsets, g.dgu, z_gu, db_gu, part, st));  // [dG | dU]^T [Z_gate | Z_up]
  MOE_TRY(outer_product(s, H, rp, g.offsets, g.do_perm, z_d, db_d, part, st));       // dO^T Z_down
  MOE_TRY(outer_product(s, rp, I, g.offsets, y_d, g.act, da_d, part, st));           // Y_down^T Act
  // The adapters' own blocks.
  auto extract = [&](int rows, int cols, const float* src, int src_rows, int src_cols, int row0, int col0,
                     float* dst) {
    const int64_t total4 = static_cast<int64_t>(E) * rows * cols / 4;
    extract_kernel<<<static_cast<unsigned>(ceil_div64(total4, kThreads)), kThreads, 0, st>>>(
        total4, rows, cols, src, src_rows, src_cols, row0, col0, dst);
    return hipGetLastError();
  };
  MOE_TRY(extract(I, r, db_gu, 2 * I, 2 * rp, 0, 0, g.db_gate));
  MOE_TRY(extract(I, r, db_gu, 2 * I, 2 * rp, I, rp, g.db_up));
  if (padded) {
    MOE_TRY(extract(r, H, da_g, rp, H, 0, 0, g.da_gate));
    MOE_TRY(extract(r, H, da_u, rp, H, 0, 0, g.da_up));
    MOE_TRY(extract(r, I, da_d, rp, I, 0, 0, g.da_down));
    MOE_TRY(extract(H, r, db_d, H, rp, 0, 0, g.db_down));
  }
#undef MOE_TRY
  return hipSuccess;
}

}  // namespace moe
