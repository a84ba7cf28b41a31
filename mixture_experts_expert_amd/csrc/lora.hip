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
// projections X (sA)^T and dY (sB) in one launch of proj_kernel, and the
// outer products over each expert's rows in two launches of outer_kernel,
// which write the adapter gradients in place. The frozen weights get no
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

// Adapter-gradient outer products: for each expert e, over its sorted rows p,
//   D[i][j] = sum_p L[p][l0 + i] S[p][s0 + j],  i < nl (the long side: I or
//   H columns), j < ns (the rank side, ns <= 32 NB),
// written as out[e][i][j] (dB: [nl][ns]) or, with TRANS, as out[e][j][i]
// (dA: [ns][nl]); with out1, rows j >= ns1 of a TRANS job go to out1 instead
// (row j - ns1), so that [dA_gate; dA_up] come out of one pass over x_perm.
// Only the blocks the adapters need are computed (no padded or off-diagonal
// outputs) and the results land in place, fp32 from fp32 sums.
//
// Tile: 128 long-side columns of one expert x the whole rank side, 4
// wavefronts of 32 long-side columns. The reduction runs over the expert's
// rows in chunks of 64: each thread loads 16-byte pieces (8 consecutive
// columns of one row) and writes them to LDS as they are ([row][column]);
// the matrix-core fragments (8 consecutive rows of one column) come out of
// transposed LDS reads (frag_tr); two chunks are in flight. MFMA rows are chosen so that a
// lane ends with four consecutive output elements of one output row (the
// rank side for dB, the long side for dA): 16-byte stores. The tile list is
// static (every expert, rows or not, gets its tiles: an expert without rows
// writes zeros).
constexpr int kOC = 64;         // rows per reduction chunk
// LDS rows of a chunk ([row][column], as loaded): 128 long-side columns, or
// 32 NB rank-side columns, padded so that a row's stride is 16 or 48 dwords
// mod 64: the four rows of a transposed read group then fall on disjoint banks.
constexpr int kOLw = 128 + 32;  // bf16 per long-side row (80 dwords)
__host__ __device__ constexpr int orow_s(int nb) { return 32 * nb + (nb % 2 == 1 ? 0 : 32); }
typedef short v4i16o __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16o lds_v4i16o;

// MFMA fragment (8 consecutive rows k of one column) of a [row][column] LDS
// tile through two ds_read_b64_tr_b16: lane l addresses row 8 (l/32) +
// (l%16)/4 and columns 4 (l%4) .. + 3 of the 16-column half (l/16)%2 of the
// 32-column block at col0; within each 16 lanes the read hands lane i
// element i%4 of the pieces that lanes 4j + i/4 address, so lane l ends with
// rows 8 (l/32) .. + 3 of column col0 + l%32, and the second read (4 rows
// on) with the next four.
__device__ __forceinline__ bf16x8 frag_tr(const bf16_t* tile, int row_elems, int row0, int col0, int lane) {
  const int g16 = lane >> 4, i16 = lane & 15;
  const int k = row0 + 8 * (g16 >> 1) + (i16 >> 2);
  const int col = col0 + 16 * (g16 & 1) + 4 * (i16 & 3);
  const bf16_t* p = tile + k * row_elems + col;
  const v4i16o lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16o*)(p));
  const v4i16o hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16o*)(p + 4 * row_elems));
  const v4i16o both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, both);
}

struct OuterJob {
  const bf16_t* L;  // [T*k][ldl], columns l0 .. l0 + nl
  const bf16_t* S;  // [T*k][lds], columns s0 .. s0 + ns
  float* out;       // per expert nl * ns floats (out1: the rows j >= ns1 of a TRANS job)
  float* out1;
  int ldl, l0, nl, lds, s0, ns, ns1, rows1;  // rows1: rows of out / out1 per expert (TRANS)
};
struct OuterJobs {
  OuterJob job[3];
  int n;
};

template <int NB, bool TRANS>
__global__ __launch_bounds__(kThreads) void outer_kernel(int E, const int32_t* __restrict__ offsets, OuterJobs jobs) {
  constexpr int kOS = orow_s(NB);
  __shared__ __attribute__((aligned(16))) bf16_t lt[2][kOC * kOLw];
  __shared__ __attribute__((aligned(16))) bf16_t st[2][kOC * kOS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  // Static tile list: job-major, then expert, then 128-column block.
  int t = blockIdx.x, jb = 0;
  for (; jb < jobs.n; ++jb) {
    const int nt = E * ((jobs.job[jb].nl + 127) / 128);
    if (t < nt) break;
    t -= nt;
  }
  if (jb >= jobs.n) return;  // uniform over the block
  const OuterJob& J = jobs.job[jb];
  const int tpe = (J.nl + 127) / 128;
  const int e = t / tpe, i0 = (t - e * tpe) * 128;
  const int r0 = offsets[e], rows = offsets[e + 1] - r0;

  // Pieces of a chunk: L: row q / 16, columns i0 + 8 (q % 16) .. + 7; S: row
  // q / (4 NB), columns 8 (q % (4 NB)) .. + 7. Columns past the window read
  // zeros (out of range); rows past the expert's fall outside the buffer range.
  constexpr int PL = kOC * 16 / kThreads, PS = kOC * 4 * NB / kThreads;
  uint32_t ol[PL], os[PS];
#pragma unroll
  for (int u = 0; u < PL; ++u) {
    const int q = tid + kThreads * u, c = i0 + 8 * (q & 15);
    ol[u] = c < J.nl ? 2u * static_cast<uint32_t>((q >> 4) * J.ldl + J.l0 + c) : kOutOfRange;
  }
#pragma unroll
  for (int u = 0; u < PS; ++u) {
    const int q = tid + kThreads * u, c = 8 * (q % (4 * NB));
    os[u] = c < J.ns ? 2u * static_cast<uint32_t>((q / (4 * NB)) * J.lds + J.s0 + c) : kOutOfRange;
  }
  const bf16_t* lbase = J.L + static_cast<int64_t>(r0) * J.ldl;
  const bf16_t* sbase = J.S + static_cast<int64_t>(r0) * J.lds;
  uint4 pl[2][PL], ps[2][PS];
  auto load_chunk = [&](int c, uint4 (&ql)[PL], uint4 (&qs)[PS]) __attribute__((always_inline)) {
    const int p0 = c * kOC;
    const bool live = p0 < rows;
    const int left = live ? min(rows - p0, kOC) : 0;  // the rows this chunk can address
    const rsrc_t rl = make_rsrc(lbase + (live ? static_cast<int64_t>(p0) * J.ldl : 0), 2 * left * J.ldl);
    const rsrc_t rs = make_rsrc(sbase + (live ? static_cast<int64_t>(p0) * J.lds : 0), 2 * left * J.lds);
#pragma unroll
    for (int u = 0; u < PL; ++u) ql[u] = load16(rl, ol[u]);
#pragma unroll
    for (int u = 0; u < PS; ++u) qs[u] = load16(rs, os[u]);
  };
  auto store_chunk = [&](int buf, const uint4 (&ql)[PL], const uint4 (&qs)[PS]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PL; ++u) {
      const int q = tid + kThreads * u;
      *reinterpret_cast<uint4*>(&lt[buf][(q >> 4) * kOLw + 8 * (q & 15)]) = ql[u];
    }
#pragma unroll
    for (int u = 0; u < PS; ++u) {
      const int q = tid + kThreads * u;
      *reinterpret_cast<uint4*>(&st[buf][(q / (4 * NB)) * kOS + 8 * (q % (4 * NB))]) = qs[u];
    }
  };

  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};
  // Same pipeline as proj_kernel: LDS holds chunk c, one register set chunk
  // c + 1, the other takes chunk c + 2; the chunk count is rounded up to even
  // (a chunk past the rows is all zeros).
  const int nch = ((rows + kOC - 1) / kOC + 1) & ~1;
  load_chunk(0, pl[0], ps[0]);
  load_chunk(1, pl[1], ps[1]);
  store_chunk(0, pl[0], ps[0]);
  lds_barrier();
  auto step = [&](int c, uint4 (&nl_)[PL], uint4 (&ns_)[PS], uint4 (&cl)[PL], uint4 (&cs)[PS])
      __attribute__((always_inline)) {
    const int buf = c & 1;
    load_chunk(c + 2, nl_, ns_);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sl = 0; sl < kOC / 16; ++sl) {
      const bf16x8 fl = frag_tr(lt[buf], kOLw, 16 * sl, wave * 32, lane);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 fs = frag_tr(st[buf], kOS, 16 * sl, nb * 32, lane);
        if constexpr (TRANS) acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl, fs, acc[nb], 0, 0, 0);
        else acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fs, fl, acc[nb], 0, 0, 0);
      }
    }
    store_chunk(buf ^ 1, cl, cs);
    lds_barrier();
  };
  for (int c = 0; c < nch; c += 2) {
    step(c, pl[0], ps[0], pl[1], ps[1]);
    step(c + 1, pl[1], ps[1], pl[0], ps[0]);
  }

  // Lane l holds D[8q + 4(l/32) + u][l%32], u < 4, of each 32 x 32 block nb.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = make_float4(acc[nb][4 * q], acc[nb][4 * q + 1], acc[nb][4 * q + 2], acc[nb][4 * q + 3]);
      const int a = 8 * q + 4 * h;  // first of four consecutive MFMA rows
      if constexpr (TRANS) {
        // MFMA rows: long side i; columns: rank side j.
        const int i = i0 + wave * 32 + a, j = nb * 32 + l32;
        if (i >= J.nl || j >= J.ns) continue;
        const bool second = j >= J.ns1;
        const int jr = second ? j - J.ns1 : j;  // row of out or out1
        if (jr >= J.rows1) continue;
        float* dst = (second ? J.out1 : J.out) + (static_cast<int64_t>(e) * J.rows1 + jr) * J.nl;
        *reinterpret_cast<float4*>(dst + i) = v;
      } else {
        // MFMA rows: rank side j; columns: long side i.
        const int j = nb * 32 + a, i = i0 + wave * 32 + l32;
        if (i >= J.nl || j >= J.ns) continue;
        *reinterpret_cast<float4*>(J.out + (static_cast<int64_t>(e) * J.nl + i) * J.ns + j) = v;
      }
    }
}

template <bool TRANS>
hipError_t outer_products(int E, int nb, const int32_t* offsets, const OuterJobs& jobs, hipStream_t st) {
  int tiles = 0;
  for (int j = 0; j < jobs.n; ++j) tiles += E * ((jobs.job[j].nl + 127) / 128);
  if (tiles == 0) return hipSuccess;
  switch (nb) {
    case 1: outer_kernel<1, TRANS><<<tiles, kThreads, 0, st>>>(E, offsets, jobs); break;
    case 2: outer_kernel<2, TRANS><<<tiles, kThreads, 0, st>>>(E, offsets, jobs); break;
    case 3: outer_kernel<3, TRANS><<<tiles, kThreads, 0, st>>>(E, offsets, jobs); break;
    case 4: outer_kernel<4, TRANS><<<tiles, kThreads, 0, st>>>(E, offsets, jobs); break;
    case 8: outer_kernel<8, TRANS><<<tiles, kThreads, 0, st>>>(E, offsets, jobs); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int lora_padded_rank(int r) { return (r + 63) & ~63; }

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
  const int E = s.E, H = s.H, I = s.I, rp = lora_padded_rank(r);
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
  // Outer products over each expert's rows, straight into the adapter
  // gradients: dB_gate = dG^T Z_gate, dB_up = dU^T Z_up, dB_down = dO^T
  // Z_down; then [dA_gate; dA_up] = [Y_gate | Y_up]^T X (one pass over
  // x_perm) and dA_down = Y_down^T Act.
  {
    const bf16_t* dgu = static_cast<const bf16_t*>(g.dgu);
    OuterJobs ob{};
    ob.job[0] = {dgu, static_cast<const bf16_t*>(z_gu), g.db_gate, nullptr, 2 * I, 0, I, 2 * rp, 0, r, r, r};
    ob.job[1] = {dgu, static_cast<const bf16_t*>(z_gu), g.db_up, nullptr, 2 * I, I, I, 2 * rp, rp, r, r, r};
    ob.job[2] = {static_cast<const bf16_t*>(g.do_perm), static_cast<const bf16_t*>(z_d), g.db_down, nullptr, H, 0,
                 H, rp, 0, r, r, r};
    ob.n = 3;
    MOE_TRY(outer_products<false>(E, (r + 31) / 32, g.offsets, ob, st));
    OuterJobs oa{};
    oa.job[0] = {static_cast<const bf16_t*>(g.x_perm), static_cast<const bf16_t*>(y_gu), g.da_gate, g.da_up, H, 0,
                 H, 2 * rp, 0, 2 * rp, rp, r};
    oa.job[1] = {static_cast<const bf16_t*>(g.act), static_cast<const bf16_t*>(y_d), g.da_down, nullptr, I, 0, I, rp,
                 0, r, r, r};
    oa.n = 2;
    MOE_TRY(outer_products<true>(E, 2 * rp / 32, g.offsets, oa, st));
  }
#undef MOE_TRY
  return hipSuccess;
}

}  // namespace moe
