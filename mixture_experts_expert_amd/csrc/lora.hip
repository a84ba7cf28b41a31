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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
constexpr int kMergeRowTiles = 8; // most row tiles per merge block (an expert's tiles are split evenly over blocks)
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
// Block: 128 columns of expert blockIdx.z and `per` consecutive tiles of
// 128 rows (fewer in the last block), per = the expert's ceil(N / 128)
// tiles spread evenly over ceil(tiles / kMergeRowTiles) blocks; 4
// wavefronts, each 64 columns x 64 rows of a tile (2 x 2 MFMA blocks of
// 32 x 32). MFMA rows are weight columns: the operand is A^T,
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
//
// WF (the frozen W's format): kBf16; kE4M3, codes [E][N][K] with one E8M0
// scale per row (w8 [E][N], 2^(c - 127)); kMxfp4, E2M1 codes two per byte
// [E][N][K/2] (even element in the low nibble) with one E8M0 scale per 32
// elements of a row (w8 [E][N][K/32]). Each element is decoded to fp32
// (exact) and multiplied by its scale (exact) before the add, so W' =
// bf16(deq(W) + s B A) with the same single rounding as the bf16 form.
enum WFormat : int { kBf16 = 0, kE4M3 = 1, kMxfp4 = 2 };

// E8M0 scale byte c -> 2^(c - 127) as a float for gfx950's scaled
// conversions (v_cvt_scalef32_pk_f32_fp4 / _fp8: two elements per
// instruction, multiplied by the scale exactly); c = 0 (2^-127, below the
// normal range) gives 2^-126 and the caller halves the results. An in-bounds
// GPU check against a CPU decode of every code at scales 2^-126 .. 2^127
// found them exact, E4M3's NaN codes included.
__device__ __forceinline__ float e8m0_scale(int c) {
  const int b = c & 0xff;
  return __uint_as_float(static_cast<uint32_t>(b == 0 ? 1 : b) << 23);
}

template <int NS, int WF>
__global__ __launch_bounds__(kThreads) void merge_kernel(int N, int K, int r, float s, const void* wv_in,
                                                         const uint8_t* __restrict__ w8,
                                                         const bf16_t* __restrict__ a, const bf16_t* __restrict__ b,
                                                         bf16_t* w_out, int per) {
  const bf16_t* w = static_cast<const bf16_t*>(wv_in);
  __shared__ __attribute__((aligned(16))) float lds[kMT * kStageRow];
  bf16_t* at = reinterpret_cast<bf16_t*>(lds);  // A^T [128][kLdsRow], then the fp32 stage [128][kStageRow]
  const int e = blockIdx.z;
  const int c0 = blockIdx.x * kMT, nbeg = blockIdx.y * kMT * per;
  const int nend = min(N, nbeg + kMT * per);  // this block's rows
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
  // W row runs of the current and the next row tile: 8 bf16 (16 bytes), 8
  // E4M3 codes (8 bytes) or 8 E2M1 codes (4 bytes) per thread and pass, and
  // the scale of the row (E4M3) or of the row's 32-element block (E2M1).
  typedef std::conditional_t<WF == kBf16, uint4, std::conditional_t<WF == kE4M3, uint2, uint32_t>> WRun;
  WRun wv[2][kMT / 16];
  int wsc[2][kMT / 16];
  const uint8_t* w_codes = static_cast<const uint8_t*>(wv_in);
  const rsrc_t rw = WF == kE4M3   ? make_rsrc(w_codes + wbase, N * K)
                    : WF == kMxfp4 ? make_rsrc(w_codes + wbase / 2, N * (K / 2))
                                   : make_rsrc(w + wbase, 2 * N * K);
  const int nsc = WF == kE4M3 ? N : (WF == kMxfp4 ? N * (K / 32) : 0);  // scales of one expert
  const rsrc_t rsc = make_rsrc(w8 + (WF == kBf16 ? 0 : static_cast<int64_t>(e) * nsc), nsc);
  const rsrc_t rb = make_rsrc(be, 2 * N * r);
  auto load_tile = [&](int nt, WRun (&wt)[kMT / 16], int (&sc)[kMT / 16]) __attribute__((always_inline)) {
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
      if constexpr (WF == kE4M3) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rw, cok ? static_cast<uint32_t>(n * K + c0 + rcol)
                                                                     : kOutOfRange, 0, 0);
        wt[q] = make_uint2(v.x, v.y);
        sc[q] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b8(rsc, static_cast<uint32_t>(n), 0, 0));
      } else if constexpr (WF == kMxfp4) {
        wt[q] = __builtin_amdgcn_raw_buffer_load_b32(rw, cok ? static_cast<uint32_t>(n * K + c0 + rcol) / 2
                                                             : kOutOfRange, 0, 0);
        sc[q] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b8(
            rsc, cok ? static_cast<uint32_t>(n * (K / 32) + (c0 + rcol) / 32) : kOutOfRange, 0, 0));
      } else {
        wt[q] = load16(rw, cok ? 2u * static_cast<uint32_t>(n * K + c0 + rcol) : kOutOfRange);
        sc[q] = 0;
      }
    }
  };
  // One row tile at nt with its W runs in (wc_t, sc_t); the next tile's
  // loads go to (wn_t, sn_t). Past the block's rows they address rows >= N,
  // which read zeros without touching memory: no branch, so the compiler
  // keeps the loads in flight across the epilogue's waits.
  auto row_tile = [&](int nt, const WRun (&wc_t)[kMT / 16], const int (&sc_t)[kMT / 16], WRun (&wn_t)[kMT / 16],
                      int (&sn_t)[kMT / 16]) __attribute__((always_inline)) {
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
    load_tile(nt + kMT < nend ? nt + kMT : N, wn_t, sn_t);
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
#pragma unroll
    for (int q = 0; q < kMT / 16; ++q) {
      const int n = nt + 16 * q + rrow;
      if (n >= N || !cok) continue;
      const float* sp = &lds[(16 * q + rrow) * kStageRow + rcol];
      const float4 v0 = *reinterpret_cast<const float4*>(sp), v1 = *reinterpret_cast<const float4*>(sp + 4);
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      float wf[8];
      if constexpr (WF == kMxfp4) {
        // The block's E8M0 scale applied by the conversion itself (exact:
        // a power of two); the element at byte j's low nibble comes first.
        const float sc = e8m0_scale(sc_t[q]);
        const uint32_t c8 = wc_t[q];
        const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c8, sc, 0);
        const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c8, sc, 1);
        const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c8, sc, 2);
        const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c8, sc, 3);
        wf[0] = v0.x, wf[1] = v0.y, wf[2] = v1.x, wf[3] = v1.y;
        wf[4] = v2.x, wf[5] = v2.y, wf[6] = v3.x, wf[7] = v3.y;
        if ((sc_t[q] & 0xff) == 0) {  // 2^-127 is below the normal range: 2^-126, then halved (exact)
#pragma unroll
          for (int p = 0; p < 8; ++p) wf[p] *= 0.5f;
        }
      } else if constexpr (WF == kE4M3) {
        const float sc = e8m0_scale(sc_t[q]);  // the row's E8M0 scale
        const uint32_t c2[2] = {wc_t[q].x, wc_t[q].y};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c2[p], sc, false);
          const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c2[p], sc, true);
          wf[4 * p] = lo.x;
          wf[4 * p + 1] = lo.y;
          wf[4 * p + 2] = hi.x;
          wf[4 * p + 3] = hi.y;
        }
        if ((sc_t[q] & 0xff) == 0) {
#pragma unroll
          for (int p = 0; p < 8; ++p) wf[p] *= 0.5f;
        }
      } else {
        const uint32_t win[4] = {wc_t[q].x, wc_t[q].y, wc_t[q].z, wc_t[q].w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          wf[2 * p] = __uint_as_float(win[p] << 16);
          wf[2 * p + 1] = __uint_as_float(win[p] & 0xffff0000u);
        }
      }
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float lo = wf[2 * p] + s * v[2 * p];
        const float hi = wf[2 * p + 1] + s * v[2 * p + 1];
        o[p] = pack_bf16x2(lo, hi);
      }
      *reinterpret_cast<uint4*>(w_out + wbase + static_cast<int64_t>(n) * K + c0 + rcol) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
  };
  // Row tiles two at a time, so that the two register sets of W runs stay
  // compile-time named.
  load_tile(nbeg, wv[0], wsc[0]);
  for (int nt = nbeg; nt < nend; nt += 2 * kMT) {
    row_tile(nt, wv[0], wsc[0], wv[1], wsc[1]);
    if (nt + kMT < nend) row_tile(nt + kMT, wv[1], wsc[1], wv[0], wsc[0]);
  }
}

__device__ __forceinline__ uint32_t scale_pair(uint32_t v, float s) {
  const float lo = s * __uint_as_float(v << 16), hi = s * __uint_as_float(v & 0xffff0000u);
  return pack_bf16x2(lo, hi);
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
      o[p] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(J) * nb * C) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Rank-wide projections: out[p][n] = sum_k rows[p][k] W[e][n][k] over each
// expert e's sorted rows p, W [E][N][K], N a multiple of 32 up to 32 NB,
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
  const bf16_t* rows;  // [T*k][K], or [nsrc][K] read through tok
  const bf16_t* w;     // [E][N][K]
  bf16_t* out;         // [T*k][N]
  int K, N;
  const int32_t* tok;  // optional: sorted row p reads row tok[p] of rows
  const float* rw;     // optional: output row p scaled by rw[p] (fp32, before rounding)
  int nsrc;            // rows of `rows` when gathered
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
  // Gathered rows: the range covers the whole source, and each lane's row
  // offset comes from the row's token (rows past the valid ones get an
  // offset outside the range).
  const bool gathered = J.tok != nullptr;
  const bf16_t* abase = gathered ? rows : rows + static_cast<int64_t>(r0) * K;
  const int arows = gathered ? J.nsrc : valid;
  const bf16_t* wbase = w + static_cast<int64_t>(e) * N * K;
  // 16-byte pieces of a chunk: piece q is row q / 8, bytes 16 (q % 8) of its 128.
  constexpr int PA = kPR * 8 / kThreads, PB = NMAX * 8 / kThreads;
  uint32_t oa[PA], ob[PB];
#pragma unroll
  for (int i = 0; i < PA; ++i) {
    const int q = tid + kThreads * i, row = q >> 3;
    if (gathered) {
      const rsrc_t rt = make_rsrc(J.tok + r0, 4 * valid);
      const int t = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(rt, 4u * row, 0, 0));
      oa[i] = row < valid ? 2u * static_cast<uint32_t>(t * K) + 16u * (q & 7) : kOutOfRange;
    } else {
      oa[i] = 2u * static_cast<uint32_t>(row * K) + 16u * (q & 7);
    }
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
    const rsrc_t ra = make_rsrc(abase + (live ? k0 : 0), live ? 2 * (arows * K - k0) : 0);
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
  const float rwt = J.rw != nullptr && row < valid ? J.rw[r0 + row] : 1.0f;
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
      if (J.rw != nullptr) {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] *= rwt;
      }
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
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
    case 2: proj_kernel<2><<<grid, kThreads, 0, st>>>(s.E, offsets, jobs); break;
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
// rank side for dB, the long side for dA): 16-byte stores. Every expert,
// rows or not, gets its tiles (an expert without rows writes zeros).
//
// Long experts are split: the launch is persistent (one block per CU), and
// an expert whose row chunks exceed cap = max(kOuterMinChunks, W / (2 grid))
// (W the launch's total work in chunk-tiles) has its rows cut into
// ceil(chunks / cap) pieces of about equal length, each a tile of its own.
// Piece 0 writes the gradient; later pieces write fp32 partial tiles to the
// workspace, which outer_reduce_kernel adds in piece order afterwards (no
// atomics: the result does not depend on timing). Under skewed routing the
// few experts holding a large share of the rows then no longer leave their
// tiles running long after the others.
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
  const bf16_t* L;  // [T*k][ldl], columns l0 .. l0 + nl (or [lsrc][ldl] read through ltok)
  const bf16_t* S;  // [T*k][lds], columns s0 .. s0 + ns
  float* out;       // per expert nl * ns floats (out1: the rows j >= ns1 of a TRANS job)
  float* out1;
  int ldl, l0, nl, lds, s0, ns, ns1, rows1;  // rows1: rows of out / out1 per expert (TRANS)
  const int32_t* ltok;  // optional: sorted row p of L is row ltok[p] of L
  int lsrc;             // rows of L
};
struct OuterJobs {
  OuterJob job[3];
  int n;
};

constexpr int kOuterMinChunks = 16;     // a piece of a split expert: at least 16 chunks of 64 rows

// Persistent grid of the outer products: one block per compute unit.
int outer_grid() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    cached = cus;
  }
  return cached;
}
constexpr int kOuterPartFloats = 128 * 256;  // one partial tile (128 long-side x up to 256 rank-side)

// The split plan, made once per launch by outer_plan_kernel (one block) into
// the workspace. Expert e has chunks(e) = ceil(rows / kOC) row chunks and
// pieces(e) = ceil(chunks / cap) when chunks > cap (else 1), each piece of
// ceil(chunks / pieces) chunks; a tile is (expert, piece, job, 128-column
// block). The experts are taken longest first (so the split ones come first
// and the hardware starts the longest tiles earliest); tile t of the launch
// is piece g = t / tpe of that order, column index t % tpe over the jobs'
// column blocks (tpe of them). A later piece of a split expert writes a
// partial tile (slot) and each (split expert, job, column block) is a unit
// of the reduction, which adds its pieces' slots in piece order.
struct OuterDesc {
  int job, e, piece, pieces, cb, slot;
};
struct OuterUnit {
  int job, e, cb, slot1, pieces;  // piece p >= 1 in slot slot1 + (p - 1) tpe
};
__device__ __forceinline__ int outer_pieces(int steps, int cap) { return steps > cap ? (steps + cap - 1) / cap : 1; }

constexpr int kPlanThreads = 1024;  // one expert per thread (E <= 1024)

// Block-wide exclusive scan of v (thread q) into out[0 .. n] (out[n] the
// total): a wavefront scan through shuffles, then the wavefronts' totals.
__device__ __forceinline__ void plan_scan(int v, int* out, int* wtot, int n, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(incl, o, 64);
    if (lane >= o) incl += x;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    before += w < wave ? wtot[w] : 0;
    total += wtot[w];
  }
  if (tid < n) out[tid] = before + incl - v;
  if (tid == 0) out[n] = total;
  __syncthreads();  // out complete; wtot free for the next scan
}

// Largest q < n with a[q] <= v (a non-decreasing, a[0] <= v).
__device__ __forceinline__ int plan_find(const int* a, int n, int v) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= v) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Job and column block of column index c (< tpe) over the jobs.
__device__ __forceinline__ void plan_column(const OuterJobs& jobs, int c, int& job, int& cb) {
  job = 0;
  for (; job < jobs.n - 1; ++job) {
    const int n = (jobs.job[job].nl + 127) / 128;
    if (c < n) break;
    c -= n;
  }
  cb = c;
}

// hdr[0] = tiles, hdr[1] = reduction units; desc [tiles], units [units].
__global__ __launch_bounds__(kPlanThreads) void outer_plan_kernel(int E, const int32_t* __restrict__ offsets,
                                                                  OuterJobs jobs, int grid, int* __restrict__ hdr,
                                                                  OuterDesc* __restrict__ desc,
                                                                  OuterUnit* __restrict__ units) {
  __shared__ int key[kPlanThreads], order[kPlanThreads], wtot[kPlanThreads / 64];
  __shared__ int pst[kPlanThreads + 1], qst[kPlanThreads + 1], sst[kPlanThreads + 1];
  const int tid = threadIdx.x;
  const int chunks = tid < E ? (offsets[tid + 1] - offsets[tid] + kOC - 1) / kOC : 0;
  // Experts by chunk count, descending, ties to the lower index: expert e's
  // position is the number of keys above its own.
  const int mykey = chunks * 2048 + (2047 - tid);
  key[tid] = mykey;
  plan_scan(chunks, pst, wtot, E, tid);  // (its barriers publish key too)
  int tpe = 0;
  for (int j = 0; j < jobs.n; ++j) tpe += (jobs.job[j].nl + 127) / 128;
  // cap >= work / (2 grid): fewer than 2 grid partial tiles at any shape
  const int64_t work = static_cast<int64_t>(tpe) * max(pst[E], E);
  const int cap = max(kOuterMinChunks, static_cast<int>((work + 2 * grid - 1) / (2 * grid)));
  if (tid < E) {
    int pos = 0;
    for (int q = 0; q < E; ++q) pos += key[q] > mykey ? 1 : 0;
    order[pos] = tid;
  }
  __syncthreads();
  // From here on, thread q stands for the expert at position q.
  const int eq = tid < E ? order[tid] : 0;
  const int cq = tid < E ? (offsets[eq + 1] - offsets[eq] + kOC - 1) / kOC : 0;
  const int pieces = tid < E ? outer_pieces(cq, cap) : 0;
  plan_scan(pieces, pst, wtot, E, tid);
  plan_scan(tid < E ? pieces - 1 : 0, qst, wtot, E, tid);
  plan_scan(pieces > 1 ? 1 : 0, sst, wtot, E, tid);  // the split experts: the first sst[E] positions
  const int tiles = pst[E] * tpe, nunits = sst[E] * tpe;
  for (int t = tid; t < tiles; t += kPlanThreads) {
    const int g = t / tpe, c = t - g * tpe;
    const int q = plan_find(pst, E, g);
    const int np = pst[q + 1] - pst[q], p = g - pst[q];
    int job, cb;
    plan_column(jobs, c, job, cb);
    desc[t] = OuterDesc{job, order[q], p, np, cb, p > 0 ? (qst[q] + p - 1) * tpe + c : -1};
  }
  for (int u = tid; u < nunits; u += kPlanThreads) {
    const int q = u / tpe, c = u - q * tpe;
    int job, cb;
    plan_column(jobs, c, job, cb);
    units[u] = OuterUnit{job, order[q], cb, qst[q] * tpe + c, pst[q + 1] - pst[q]};
  }
  if (tid == 0) {
    hdr[0] = tiles;
    hdr[1] = nunits;
  }
}

template <int NB, bool TRANS>
__global__ __launch_bounds__(kThreads) void outer_kernel(int E, const int32_t* __restrict__ offsets, OuterJobs jobs,
                                                         const int* __restrict__ hdr,
                                                         const OuterDesc* __restrict__ descs,
                                                         float* __restrict__ part) {
  constexpr int kOS = orow_s(NB);
  __shared__ __attribute__((aligned(16))) bf16_t lt[2][kOC * kOLw];
  __shared__ __attribute__((aligned(16))) bf16_t st[2][kOC * kOS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  if (static_cast<int>(blockIdx.x) >= hdr[0]) return;  // uniform over the block
  const OuterDesc d = descs[blockIdx.x];
  const OuterJob& J = jobs.job[d.job];
  const int e = d.e, i0 = d.cb * 128;
  (void)E;
  // The piece's rows: pieces of ceil(chunks / pieces) chunks each (the last
  // one may be shorter, or empty: it then writes zeros).
  const int eb = offsets[e], erows = offsets[e + 1] - eb;
  const int per = ((erows + kOC - 1) / kOC + d.pieces - 1) / d.pieces;
  const int first = d.piece * per * kOC;
  const int r0 = eb + min(first, erows);
  const int rows = max(0, min(erows, first + per * kOC) - first);
  float* const pdst = d.slot >= 0 ? part + static_cast<int64_t>(d.slot) * kOuterPartFloats : nullptr;
  // Pieces of a chunk: L: row q / 16, columns i0 + 8 (q % 16) .. + 7; S: row
  // q / (4 NB), columns 8 (q % (4 NB)) .. + 7. Columns past the window read
  // zeros (out of range); rows past the piece's fall outside the S buffer
  // range and get an L offset outside L's range. L is addressed by source
  // row: the sorted row itself, or its token (read two chunks ahead of the
  // loads that use it, so that waiting for it waits for nothing newer).
  constexpr int PL = kOC * 16 / kThreads, PS = kOC * 4 * NB / kThreads;
  uint32_t lcol[PL], os[PS];
#pragma unroll
  for (int u = 0; u < PL; ++u) {
    const int q = tid + kThreads * u, c = i0 + 8 * (q & 15);
    lcol[u] = c < J.nl ? 2u * static_cast<uint32_t>(J.l0 + c) : kOutOfRange;
  }
#pragma unroll
  for (int u = 0; u < PS; ++u) {
    const int q = tid + kThreads * u, c = 8 * (q % (4 * NB));
    os[u] = c < J.ns ? 2u * static_cast<uint32_t>((q / (4 * NB)) * J.lds + J.s0 + c) : kOutOfRange;
  }
  const rsrc_t rl = make_rsrc(J.L, 2 * J.lsrc * J.ldl);
  const rsrc_t rtok = make_rsrc(J.ltok != nullptr ? static_cast<const void*>(J.ltok + r0) : static_cast<const void*>(J.L),
                                J.ltok != nullptr ? 4 * rows : 0);
  const int tok_add = J.ltok != nullptr ? 0 : r0;  // identity rows: the token is the sorted row
  const bf16_t* sbase = J.S + static_cast<int64_t>(r0) * J.lds;
  uint4 pl[2][PL], ps[2][PS];
  int tk[2][PL];  // source rows of the chunks to load next (by chunk parity)
  auto load_tok = [&](int c, int (&t)[PL]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PL; ++u) {
      const int row = c * kOC + ((tid + kThreads * u) >> 4);
      t[u] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(rtok, 4u * static_cast<uint32_t>(row), 0, 0)) +
             tok_add + (J.ltok != nullptr ? 0 : row);
    }
  };
  auto load_chunk = [&](int c, uint4 (&ql)[PL], uint4 (&qs)[PS], int (&t)[PL]) __attribute__((always_inline)) {
    const int p0 = c * kOC;
    const bool live = p0 < rows;
    const int left = live ? min(rows - p0, kOC) : 0;  // the rows this chunk can address
    const rsrc_t rs = make_rsrc(sbase + (live ? static_cast<int64_t>(p0) * J.lds : 0), 2 * left * J.lds);
#pragma unroll
    for (int u = 0; u < PL; ++u) {
      const int row = p0 + ((tid + kThreads * u) >> 4);
      const uint32_t off = row < rows ? 2u * static_cast<uint32_t>(t[u] * J.ldl) + lcol[u] : kOutOfRange;
      ql[u] = load16(rl, lcol[u] == kOutOfRange ? kOutOfRange : off);
    }
#pragma unroll
    for (int u = 0; u < PS; ++u) qs[u] = load16(rs, os[u]);
    load_tok(c + 2, t);  // this register set's next chunk
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
  load_tok(0, tk[0]);
  load_tok(1, tk[1]);
  load_chunk(0, pl[0], ps[0], tk[0]);
  load_chunk(1, pl[1], ps[1], tk[1]);
  store_chunk(0, pl[0], ps[0]);
  lds_barrier();
  auto step = [&](int c, uint4 (&nl_)[PL], uint4 (&ns_)[PS], uint4 (&cl)[PL], uint4 (&cs)[PS], int (&tkn)[PL])
      __attribute__((always_inline)) {
    const int buf = c & 1;
    load_chunk(c + 2, nl_, ns_, tkn);
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
    step(c, pl[0], ps[0], pl[1], ps[1], tk[0]);
    step(c + 1, pl[1], ps[1], pl[0], ps[0], tk[1]);
  }

  // Lane l holds D[8q + 4(l/32) + u][l%32], u < 4, of each 32 x 32 block nb.
  // A later piece of a split expert writes its partial tile instead, in the
  // same orientation: [i - i0][j] (row 256) or, TRANS, [j][i - i0] (row 128).
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
        if (pdst) {
          *reinterpret_cast<float4*>(pdst + j * 128 + (i - i0)) = v;
          continue;
        }
        const bool second = j >= J.ns1;
        const int jr = second ? j - J.ns1 : j;  // row of out or out1
        if (jr >= J.rows1) continue;
        float* dst = (second ? J.out1 : J.out) + (static_cast<int64_t>(e) * J.rows1 + jr) * J.nl;
        *reinterpret_cast<float4*>(dst + i) = v;
      } else {
        // MFMA rows: rank side j; columns: long side i.
        const int j = nb * 32 + a, i = i0 + wave * 32 + l32;
        if (i >= J.nl || j >= J.ns) continue;
        if (pdst) {
          *reinterpret_cast<float4*>(pdst + (i - i0) * 256 + j) = v;
          continue;
        }
        *reinterpret_cast<float4*>(J.out + (static_cast<int64_t>(e) * J.nl + i) * J.ns + j) = v;
      }
    }
}

// Adds the partial tiles of a split expert into its adapter gradient, in
// piece order (piece 0 is already there): one block per reduction unit
// (job, split expert, column block) of the plan.
template <bool TRANS>
__global__ __launch_bounds__(kThreads) void outer_reduce_kernel(OuterJobs jobs, int tpe, const int* __restrict__ hdr,
                                                                const OuterUnit* __restrict__ units,
                                                                const float* __restrict__ part) {
  if (static_cast<int>(blockIdx.x) >= hdr[1]) return;  // uniform over the block
  const OuterUnit U = units[blockIdx.x];
  const OuterJob& J = jobs.job[U.job];
  const int e = U.e, i0 = U.cb * 128;
  // Four consecutive elements per thread along the contiguous side (i for
  // TRANS, j otherwise; nl and ns are multiples of 8).
  constexpr int kU = 4;  // groups per thread and pass, their loads in flight together
  const int groups = 32 * J.ns;  // 128 x ns elements
  for (int g0 = threadIdx.x; g0 < groups; g0 += kU * kThreads) {
    float* dst[kU];
    int local[kU];
    float4 sum[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int g = g0 + u * kThreads;
      dst[u] = nullptr;
      if (g >= groups) continue;
      int i, j;
      if constexpr (TRANS) {
        j = g / 32;
        i = i0 + 4 * (g - j * 32);
      } else {
        const int per = J.ns / 4;
        i = i0 + g / per;
        j = 4 * (g - (g / per) * per);
      }
      if (i >= J.nl) continue;
      if constexpr (TRANS) {
        const bool second = j >= J.ns1;
        const int jr = second ? j - J.ns1 : j;
        if (jr >= J.rows1) continue;
        dst[u] = (second ? J.out1 : J.out) + (static_cast<int64_t>(e) * J.rows1 + jr) * J.nl + i;
      } else {
        dst[u] = J.out + (static_cast<int64_t>(e) * J.nl + i) * J.ns + j;
      }
      local[u] = TRANS ? j * 128 + (i - i0) : (i - i0) * 256 + j;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (dst[u]) sum[u] = *reinterpret_cast<const float4*>(dst[u]);
    for (int p = 1; p < U.pieces; ++p) {
      const float* src = part + static_cast<int64_t>(U.slot1 + (p - 1) * tpe) * kOuterPartFloats;
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (dst[u]) {
          const float4 v = *reinterpret_cast<const float4*>(src + local[u]);
          sum[u].x += v.x;
          sum[u].y += v.y;
          sum[u].z += v.z;
          sum[u].w += v.w;
        }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (dst[u]) *reinterpret_cast<float4*>(dst[u]) = sum[u];
  }
}

// Workspace of one outer-product launch: the plan (header, tile
// descriptors, reduction units) and the partial tiles.
struct OuterSpace {
  int* hdr;
  OuterDesc* desc;
  OuterUnit* units;
  float* part;
};

template <bool TRANS>
hipError_t outer_products(int E, int nb, const int32_t* offsets, const OuterJobs& jobs, const OuterSpace& w,
                          hipStream_t st) {
  const int grid = outer_grid();
  int tiles_per_expert = 0;
  for (int j = 0; j < jobs.n; ++j) tiles_per_expert += (jobs.job[j].nl + 127) / 128;
  // At most one tile per (job, expert, column block) plus fewer than 2 grid
  // partial tiles; blocks past the plan's count return at once.
  const unsigned tiles = static_cast<unsigned>(tiles_per_expert * E + 2 * grid);
  outer_plan_kernel<<<1, kPlanThreads, 0, st>>>(E, offsets, jobs, grid, w.hdr, w.desc, w.units);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  switch (nb) {
    case 1: outer_kernel<1, TRANS><<<tiles, kThreads, 0, st>>>(E, offsets, jobs, w.hdr, w.desc, w.part); break;
    case 2: outer_kernel<2, TRANS><<<tiles, kThreads, 0, st>>>(E, offsets, jobs, w.hdr, w.desc, w.part); break;
    case 3: outer_kernel<3, TRANS><<<tiles, kThreads, 0, st>>>(E, offsets, jobs, w.hdr, w.desc, w.part); break;
    case 4: outer_kernel<4, TRANS><<<tiles, kThreads, 0, st>>>(E, offsets, jobs, w.hdr, w.desc, w.part); break;
    case 8: outer_kernel<8, TRANS><<<tiles, kThreads, 0, st>>>(E, offsets, jobs, w.hdr, w.desc, w.part); break;
    default: return hipErrorInvalidValue;
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  outer_reduce_kernel<TRANS><<<static_cast<unsigned>(2 * grid), kThreads, 0, st>>>(jobs, tiles_per_expert, w.hdr,
                                                                                      w.units, w.part);
  return hipGetLastError();
}

}  // namespace

// The projections' output width: the rank rounded up to 32, 64 or 128 (whole
// 32-column blocks of the projection tile; a rank of 8 does 4x, not 8x, its
// own work).
int lora_padded_rank(int r) { return r <= 32 ? 32 : (r <= 64 ? 64 : 128); }

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
  // Split plan and partial tiles of the outer products: at most 2 ceil(I /
  // 128) + ceil(H / 128) tiles per expert plus fewer than 2 grid partial
  // tiles (cap >= total work / (2 grid)), and fewer reduction units.
  const int64_t grid = outer_grid();
  const int64_t max_tiles = (2 * ceil_div(I, 128) + ceil_div(H, 128)) * E + 2 * grid;
  l.plan = take(256 + max_tiles * static_cast<int64_t>(sizeof(OuterDesc)) + 2 * grid * sizeof(OuterUnit));
  l.part = take(2 * grid * kOuterPartFloats * 4);
  l.total = off;
  return l;
}

namespace {
template <int WF>
hipError_t merge_launch(int E, int N, int K, int r, float s, const void* w, const uint8_t* w8, const void* a,
                        const void* b, void* w_out, hipStream_t st) {
  const int tiles = ceil_div(N, kMT), per = ceil_div(tiles, ceil_div(tiles, kMergeRowTiles));
  const dim3 grid(static_cast<unsigned>(ceil_div(K, kMT)), static_cast<unsigned>(ceil_div(tiles, per)),
                  static_cast<unsigned>(E));
  const bf16_t* ap = static_cast<const bf16_t*>(a);
  const bf16_t* bp = static_cast<const bf16_t*>(b);
  bf16_t* op = static_cast<bf16_t*>(w_out);
  switch ((r + 15) / 16) {
    case 1: merge_kernel<1, WF><<<grid, kThreads, 0, st>>>(N, K, r, s, w, w8, ap, bp, op, per); break;
    case 2: merge_kernel<2, WF><<<grid, kThreads, 0, st>>>(N, K, r, s, w, w8, ap, bp, op, per); break;
    case 3: merge_kernel<3, WF><<<grid, kThreads, 0, st>>>(N, K, r, s, w, w8, ap, bp, op, per); break;
    case 4: merge_kernel<4, WF><<<grid, kThreads, 0, st>>>(N, K, r, s, w, w8, ap, bp, op, per); break;
    case 5: merge_kernel<5, WF><<<grid, kThreads, 0, st>>>(N, K, r, s, w, w8, ap, bp, op, per); break;
    case 6: merge_kernel<6, WF><<<grid, kThreads, 0, st>>>(N, K, r, s, w, w8, ap, bp, op, per); break;
    case 7: merge_kernel<7, WF><<<grid, kThreads, 0, st>>>(N, K, r, s, w, w8, ap, bp, op, per); break;
    case 8: merge_kernel<8, WF><<<grid, kThreads, 0, st>>>(N, K, r, s, w, w8, ap, bp, op, per); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_lora_merge(int E, int N, int K, int r, float s, const void* w, const void* a, const void* b,
                             void* w_out, hipStream_t st) {
  return merge_launch<kBf16>(E, N, K, r, s, w, nullptr, a, b, w_out, st);
}

hipError_t launch_lora_merge_fp8(int E, int N, int K, int r, float s, const uint8_t* wq, const uint8_t* w8,
                                 const void* a, const void* b, void* w_out, hipStream_t st) {
  return merge_launch<kE4M3>(E, N, K, r, s, wq, w8, a, b, w_out, st);
}

hipError_t launch_lora_merge_mxfp4(int E, int N, int K, int r, float s, const uint8_t* wq, const uint8_t* w8,
                                   const void* a, const void* b, void* w_out, hipStream_t st) {
  return merge_launch<kMxfp4>(E, N, K, r, s, wq, w8, a, b, w_out, st);
}

namespace {
// The workspace's named regions.
struct LoraPtrs {
  bf16_t *sa_gu, *sa_d, *sbt_gu, *sbt_d, *z_gu, *z_d, *y_gu, *y_d;
  OuterSpace os;
};
LoraPtrs lora_ptrs(const moe_shape& s, int r, void* ws) {
  const LoraLayout l = lora_layout(s, r);
  char* base = static_cast<char*>(ws);
  auto at = [&](size_t o) { return reinterpret_cast<bf16_t*>(base + o); };
  LoraPtrs p{};
  p.sa_gu = at(l.sa_gu);
  p.sa_d = at(l.sa_d);
  p.sbt_gu = at(l.sbt_gu);
  p.sbt_d = at(l.sbt_d);
  p.z_gu = at(l.z_gu);
  p.z_d = at(l.z_d);
  p.y_gu = at(l.y_gu);
  p.y_d = at(l.y_d);
  const int64_t max_tiles = (2 * ceil_div(s.I, 128) + ceil_div(s.H, 128)) * static_cast<int64_t>(s.E) + 2 * outer_grid();
  p.os.hdr = reinterpret_cast<int*>(base + l.plan);
  p.os.desc = reinterpret_cast<OuterDesc*>(base + l.plan + 256);
  p.os.units = reinterpret_cast<OuterUnit*>(base + l.plan + 256 + max_tiles * sizeof(OuterDesc));
  p.os.part = reinterpret_cast<float*>(base + l.part);
  return p;
}
}  // namespace

#define MOE_TRY(x) \
  if ((err = (x)) != hipSuccess) return err

hipError_t launch_lora_prepare(const moe_shape& s, int r, float scale, const LoraArgs& g, void* ws, hipStream_t st) {
  const LoraPtrs p = lora_ptrs(s, r, ws);
  const int E = s.E, H = s.H, I = s.I, rp = lora_padded_rank(r);
  const bf16_t* a_gate = static_cast<const bf16_t*>(g.a_gate);
  const bf16_t* a_up = static_cast<const bf16_t*>(g.a_up);
  const bf16_t* a_down = static_cast<const bf16_t*>(g.a_down);
  const bf16_t* b_gate = static_cast<const bf16_t*>(g.b_gate);
  const bf16_t* b_up = static_cast<const bf16_t*>(g.b_up);
  const bf16_t* b_down = static_cast<const bf16_t*>(g.b_down);
  hipError_t err;
  // Scaled, stacked adapters (bf16, rounded once): sA_gu = [sA_gate; sA_up],
  // sA_d, the transposed block diagonal of sB_gate and sB_up, sB_down^T.
  stack_a_kernel<<<dim3(E * 2 * rp, ceil_div(H / 8, kThreads)), kThreads, 0, st>>>(r, rp, H, scale, a_gate, a_up,
                                                                                     p.sa_gu);
  MOE_TRY(hipGetLastError());
  stack_a_kernel<<<dim3(E * rp, ceil_div(I / 8, kThreads)), kThreads, 0, st>>>(r, rp, I, scale, a_down, nullptr,
                                                                                 p.sa_d);
  MOE_TRY(hipGetLastError());
  blockdiag_t_kernel<<<dim3(2 * I / 64, E), kThreads, 0, st>>>(I, r, rp, scale, b_gate, b_up, p.sbt_gu);
  MOE_TRY(hipGetLastError());
  blockdiag_t_kernel<<<dim3(H / 64, E), kThreads, 0, st>>>(H, r, rp, scale, b_down, nullptr, p.sbt_d);
  MOE_TRY(hipGetLastError());
  return hipSuccess;
}

hipError_t launch_lora_project(const moe_shape& s, int r, int which, const void* in, const int32_t* offsets,
                               void* ws, hipStream_t st, const int32_t* tok, const float* rw) {
  const LoraPtrs p = lora_ptrs(s, r, ws);
  const int H = s.H, I = s.I, rp = lora_padded_rank(r), M = s.T * s.k;
  const int nsrc = tok != nullptr ? s.T : M;
  const bf16_t* x = static_cast<const bf16_t*>(in);
  ProjJobs pj{};
  switch (which) {
    case 0: pj.job[0] = {x, p.sa_gu, p.z_gu, H, 2 * rp, tok, rw, nsrc}; break;
    case 1: pj.job[0] = {x, p.sbt_gu, p.y_gu, 2 * I, 2 * rp, tok, rw, nsrc}; break;
    case 2: pj.job[0] = {x, p.sa_d, p.z_d, I, rp, tok, rw, nsrc}; break;
    default: pj.job[0] = {x, p.sbt_d, p.y_d, H, rp, tok, rw, nsrc}; break;
  }
  pj.n = 1;
  return projections(s, pj.job[0].N < 64 ? 64 : pj.job[0].N, offsets, pj, st);  // the kernel's widths: 64, 128, 256
}

hipError_t launch_lora_outer(const moe_shape& s, int r, const LoraArgs& g, void* ws, hipStream_t st) {
  const LoraPtrs p = lora_ptrs(s, r, ws);
  const int E = s.E, H = s.H, I = s.I, rp = lora_padded_rank(r);
  const int32_t* tok = g.row_token;
  const int M = s.T * s.k, nsrc = tok != nullptr ? s.T : M;
  hipError_t err;
  // Outer products over each expert's rows, straight into the adapter
  // gradients: dB_gate = dG^T Z_gate, dB_up = dU^T Z_up, dB_down = dO^T
  // Z_down; then [dA_gate; dA_up] = [Y_gate | Y_up]^T X (one pass over
  // x_perm) and dA_down = Y_down^T Act.
  const bf16_t* dgu = static_cast<const bf16_t*>(g.dgu);
  OuterJobs ob{};
  ob.job[0] = {dgu, p.z_gu, g.db_gate, nullptr, 2 * I, 0, I, 2 * rp, 0, r, r, r, nullptr, M};
  ob.job[1] = {dgu, p.z_gu, g.db_up, nullptr, 2 * I, I, I, 2 * rp, rp, r, r, r, nullptr, M};
  ob.job[2] = {static_cast<const bf16_t*>(g.do_perm), p.z_d, g.db_down, nullptr, H, 0, H, rp, 0, r, r, r, tok, nsrc};
  ob.n = 3;
  MOE_TRY(outer_products<false>(E, (r + 31) / 32, g.offsets, ob, p.os, st));
  OuterJobs oa{};
  oa.job[0] = {static_cast<const bf16_t*>(g.x_perm), p.y_gu, g.da_gate, g.da_up, H, 0, H, 2 * rp, 0, 2 * rp, rp, r,
               tok, nsrc};
  oa.job[1] = {static_cast<const bf16_t*>(g.act), p.y_d, g.da_down, nullptr, I, 0, I, rp, 0, r, r, r, nullptr, M};
  oa.n = 2;
  return outer_products<true>(E, 2 * rp / 32, g.offsets, oa, p.os, st);
}

hipError_t launch_lora_grads(const moe_shape& s, int r, float scale, const LoraArgs& g, void* ws, hipStream_t st) {
  const LoraPtrs p = lora_ptrs(s, r, ws);
  const int H = s.H, I = s.I, rp = lora_padded_rank(r);
  hipError_t err;
  MOE_TRY(launch_lora_prepare(s, r, scale, g, ws, st));
  // Row projections Z = X (sA)^T, Y = dY (sB): [Z_gate | Z_up], [dG sB_gate |
  // dU sB_up], Z_down, dO sB_down.
  // With row_token, x and dy are read through the sorted rows' tokens, and
  // dO = w dy enters through the weight applied in fp32 to the two
  // projections that carry it: Z_down' = w Z_down (for dB_down = dy^T Z_down')
  // and Y_down = w (dy sB_down).
  const int32_t* tok = g.row_token;
  const float* rwt = tok != nullptr ? g.row_weight : nullptr;
  const int M = s.T * s.k, nsrc = tok != nullptr ? s.T : M;
  ProjJobs pj{};
  const bf16_t* xp = static_cast<const bf16_t*>(g.x_perm);
  pj.job[0] = {xp, p.sa_gu, p.z_gu, H, 2 * rp, tok, nullptr, nsrc};
  pj.job[1] = {static_cast<const bf16_t*>(g.dgu), p.sbt_gu, p.y_gu, 2 * I, 2 * rp, nullptr, nullptr, M};
  pj.job[2] = {static_cast<const bf16_t*>(g.act), p.sa_d, p.z_d, I, rp, nullptr, rwt, M};
  pj.job[3] = {static_cast<const bf16_t*>(g.do_perm), p.sbt_d, p.y_d, H, rp, tok, rwt, nsrc};
  pj.n = 4;
  MOE_TRY(projections(s, 2 * rp, g.offsets, pj, st));
  return launch_lora_outer(s, r, g, ws, st);
}
#undef MOE_TRY

}  // namespace moe
