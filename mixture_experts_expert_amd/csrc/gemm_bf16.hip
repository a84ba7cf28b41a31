// Grouped GEMMs of the expert stage in bf16 on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// The rows of every expert are contiguous after moe_permute (sourcepulse
// summary, "How It Works": inputs sorted by expert, grouped GEMM on
// persistent workers), so one kernel walks a device-side list of tiles:
//
//   grouped-M (forward and data gradients): a tile is up to BM rows of one
//     expert times BN output columns; the reduction runs over H, I or 2I.
//   grouped-K (weight gradients): a tile is a BM x BN block of one expert's
//     weight gradient; the reduction runs over that expert's rows, whose
//     count is ragged (0 when no token picked the expert: the tile then
//     writes zeros).
//
// Six modes share the core:
//   GATEUP       G = X W_gate^T, U = X W_up^T, A = silu(G) U     (epilogue)
//   DOWN         O = A W_down^T
//   DGRAD_DOWN   dA = dO W_down; dG, dU by the SwiGLU derivative (epilogue)
//   DGRAD_GATEUP dX = [dG | dU] [W_gate ; W_up]
//   WGRAD_DOWN   dW_down[e] = dO_e^T A_e                          (fp32 out)
//   WGRAD_GATEUP [dW_gate ; dW_up][e] = [dG | dU]_e^T X_e          (fp32 out)
//
// Tile: 256 x 256 per workgroup of 4 wavefronts (2 x 2), 128 x 128 per
// wavefront as 4 x 4 MFMA blocks of 32 x 32, accumulators in the register
// file (256 fp32 per lane); k-steps of 32. Operands go straight from global
// memory into LDS (buffer_load ... lds: each wavefront instruction fills one
// contiguous KiB, lane l at byte 16 l) through a ring of four 32 KiB stages;
// no register staging and no LDS store phase. An operand whose reduction
// index is contiguous in memory ("k-major": the forward operands, the
// data-gradient activations) sits in LDS as [row][k], 16-byte chunks
// XOR-swizzled by row, and is read with ds_read_b128. An operand whose
// reduction index is the strided one ("mn-major": the data-gradient weights,
// both weight-gradient operands) sits as [k][column] as it is in memory,
// chunks swizzled by k, and is read with ds_read_b64_tr_b16, which hands each
// lane four consecutive k of one column (within each 16-lane group, lane i
// receives element i%4 of the pieces that lanes 4j + i/4 address). Either way
// the swizzle is applied on the global side: each lane fetches the chunk
// that belongs at its fixed LDS slot.
//
// Pipeline: with one wavefront per SIMD nothing hides a stall. Loads run
// three steps ahead of the MFMAs, one load instruction after every group of
// four MFMAs (the address unit takes about 64 bytes per clock per CU; issued
// in a burst they would hold the wavefront), and each step has a single
// barrier in its middle, after which the next step's first fragments are
// read under the current step's second half. A tile's last steps load the
// next tile's first three, and the epilogue works from registers (SwiGLU in
// place: gate and up of one element share a lane; a DPP quad transpose and a
// half-wave swap turn the MFMA layout into four-row x 128-byte store runs,
// written non-temporally), so those loads land while the results go out.
// Row blocks of a short tile that hold no rows skip their MFMAs.
//
// Scheduling: one workgroup per CU, persistent. Tile i of the list belongs
// to XCD-local workgroups: the list is cut into 8 contiguous ranges, one per
// XCD (workgroup b runs on XCD b % 8), and the tiles of one expert and one
// column block sit next to each other, so the weight slice they share is
// fetched into one XCD's L2 once.
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int NT = 256;                 // threads per workgroup
constexpr int WTM = 128, WTN = 128;     // wavefront tile
constexpr int FM = WTM / 32, FN = WTN / 32;
constexpr int CH = BK / 8;              // 16-byte chunks per LDS row
constexpr int STAGE_A = BM * BK;        // bf16 elements
constexpr int STAGE_B = BN * BK;
constexpr int STAGE = STAGE_A + STAGE_B;
constexpr int GU_COLS = BN / 2;         // intermediate columns per GATEUP tile (gate + up)

constexpr int NSTAGE = 4;               // LDS ring of k-steps; loads run NSTAGE - 1 steps ahead
constexpr int LOADS = 8;                // load instructions per wavefront and k-step (4 A + 4 B)

enum Mode : int { GATEUP = 0, DOWN = 1, DGRAD_DOWN = 2, DGRAD_GATEUP = 3, WGRAD_DOWN = 4, WGRAD_GATEUP = 5 };

constexpr bool grouped_k(int m) { return m >= WGRAD_DOWN; }
constexpr bool b_kcontig(int m) { return m == GATEUP || m == DOWN; }

struct Params {
  int T, H, E, I;
  int M;               // T * k rows of the sorted operands
  const int32_t* offsets;
  const bf16_t* a;     // x_perm | act | do_perm | dgu | do_perm | dgu
  const bf16_t* b0;    // w_gate | w_down | w_down | w_gate | act | x_perm
  const bf16_t* b1;    // w_up (GATEUP, DGRAD_GATEUP)
  const bf16_t* g_in;  // DGRAD_DOWN: saved g
  const bf16_t* u_in;  // DGRAD_DOWN: saved u
  bf16_t* out0;        // g | o_perm | dgu | dx_perm
  bf16_t* out1;        // u (GATEUP)
  bf16_t* out2;        // a (GATEUP)
  bf16_t* out3;        // GATEUP with AW: a_w[p] = bf16(row_weight[p] a[p])
  float* dw0;          // dw_down | dw_gate
  float* dw1;          // dw_up
  int accumulate;
  float* part;         // weight gradients: split-K partial tiles [tile][256][256]
  // Fused gather and routing weights (both optional): GATEUP reads row p of A
  // as row row_token[p] of x [T][H] (no x_perm), WGRAD_GATEUP reads k-row p of
  // B likewise; DOWN scales output row p by row_weight[p] before rounding.
  // GATEUP with out0 == nullptr stores A only. In the backward without
  // do_perm, DGRAD_DOWN reads row p of A as row row_token[p] of dy [T][H] and
  // scales dA row p by row_weight[p] in fp32 before the SwiGLU backward, and
  // WGRAD_DOWN reads k-row p of A likewise (its B is then a_w).
  const int32_t* row_token;
  const float* row_weight;
  // fp8 (E4M3) GATEUP/DOWN of the inference forward: a, b0, b1 hold 8-bit
  // codes; sa (one per sorted row of A) and sb0, sb1 (one per row of each
  // expert's weight matrix) their power-of-two scales as E8M0 bytes.
  const uint8_t* sa;
  const uint8_t* sb0;
  const uint8_t* sb1;
  // K extended by kx (a multiple of BK) past the main reduction (KX
  // instances: GATEUP, DOWN, DGRAD_DOWN, DGRAD_GATEUP on sorted rows): A's
  // rows continue in ax [M][kx]. B's come straight from rank-kxr adapters,
  // each padded with zeros to kxp (a multiple of BK) inside the extension:
  // GATEUP, k-major, gate columns [bx0 | 0] and up columns [0 | bx1] with
  // bx0, bx1 [E][N][kxr] (kx = 2 kxp); DOWN [bx0 | 0] (kx = kxp); the data
  // gradients' k-rows bx0 [E][kxr][N] (DGRAD_DOWN, kx = kxp) or bx0 then
  // bx1 (DGRAD_GATEUP, kx = 2 kxp).
  const bf16_t* ax;
  const bf16_t* bx0;
  const bf16_t* bx1;
  int kx, kxr, kxp;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// LDS layouts of one operand stage (bf16 elements):
//   k-major  [256 rows][32 k]   chunk c of row r at r*32 + (c ^ swk(r))*8
//   mn-major [32 k][256 cols]   chunk c of row k at k*256 + (c ^ swt(k))*8
// A k-major row is 64 bytes (four chunks); the XOR with bits 2-3 of the row
// spreads the 16 rows that one ds_read_b128 pass touches over all banks.
__device__ __forceinline__ int swk(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swt(int k) { return (k & 3) << 2; }

// Operand loads go through buffer resources: a wavefront-uniform base and a
// byte range (num_records); each lane supplies a 32-bit byte offset. A lane
// whose dwords fall outside the range writes zeros, which is how reduction
// rows past an expert's last row, the padding step of an odd step count and
// prefetches past the last step are handled, without branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes, kRsrcWord3);
}
// One 16-byte chunk per lane into LDS: lane l lands at byte 16 l of the
// 1 KiB block `blk` (wavefront-uniform).
__device__ __forceinline__ void buf_to_lds16(rsrc_t r, uint32_t voff, bf16_t* blk) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)blk, 16, voff, 0, 0, 0);
}

// Workgroup barrier between k-steps. The explicit s_waitcnt before it has
// already made this wavefront's LDS traffic and needed loads complete; a
// __syncthreads() would add a release fence that also waits for the L2
// prefetches still in flight. The empty asm statements keep the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt immediates (gfx9 encoding): vmcnt in [3:0] and [15:14], expcnt in
// [6:4], lgkmcnt in [11:8]. They wait for LDS traffic and for all but the
// newest `n` vector-memory instructions (expcnt left unconstrained).
constexpr int kWaitVm8 = 0x0078;   // vmcnt(8) lgkmcnt(0)
constexpr int kWaitVm12 = 0x007C;  // vmcnt(12) lgkmcnt(0)
constexpr int kWaitVm14 = 0x007E;  // vmcnt(14) lgkmcnt(0)
constexpr int kWaitVm16 = 0x4070;  // vmcnt(16) lgkmcnt(0)
constexpr int kWaitAll = 0x0000;   // vmcnt(0) expcnt(0) lgkmcnt(0)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Four floats -> four bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  const f32x2 lo = {a, b}, hi = {c, d};
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                    __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2)));
}

// Epilogue helpers ------------------------------------------------------------

// Logistic sigmoid from the hardware base-2 exponential and reciprocal
// (v_exp_f32, v_rcp_f32; about 1 ulp each): 1 / (1 + 2^(-g log2 e)). Large
// |g| saturates cleanly to 0 or 1. The results are rounded to bf16 anyway, so
// the few ulps against an IEEE exp and divide never show.
__device__ __forceinline__ float sigmoid_fast(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// Raw-buffer loads and stores of 8 or 16 bytes per lane. A lane whose bytes
// fall outside the resource's range reads zeros and writes nothing; kNoWrite
// is an offset outside every range used here (all are below 2^31 bytes).
constexpr uint32_t kNoWrite = 0x80000000u;
// Results are streamed out (non-temporal): the next kernel reads them from
// memory anyway, and lines left dirty in the L2 slow that read down.
constexpr int kStoreNT = 2;
__device__ __forceinline__ u32x2 load_b64(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ u32x4 load_b128(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void store_b64(u32x2 v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kStoreNT);
}
__device__ __forceinline__ void store_b128(u32x4 v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kStoreNT);
}

__device__ __forceinline__ u32x2 pack_bf16x4v(const float (&v)[4]) {
  return u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Lane exchanges inside each quad of lanes (DPP quad_perm [1,0,3,2] and
// [2,3,0,1]): the value of lane l ^ 1, of lane l ^ 2.
// Every lane of a quad has a valid source, so no "old" value is needed.
__device__ __forceinline__ uint32_t quad_swap1(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ uint32_t quad_swap2(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_swap1f(float v) { return __uint_as_float(quad_swap1(__float_as_uint(v))); }
__device__ __forceinline__ float quad_swap2f(float v) { return __uint_as_float(quad_swap2(__float_as_uint(v))); }

// 4 x 4 transpose across each quad of lanes. On entry lane c (= lane % 4)
// holds column c of rows 0..3 in v[0..3]; on exit it holds row c, columns
// 0..3. The first exchange pairs lanes across bit 1 (each keeps rows 0-1 or
// rows 2-3, of columns c%2 and c%2 + 2), the second across bit 0.
__device__ __forceinline__ void quad_transpose(float (&v)[4], int lane) {
  const bool c1 = (lane & 2) != 0, c0 = (lane & 1) != 0;
  const float x0 = quad_swap2f(c1 ? v[0] : v[2]);
  const float x1 = quad_swap2f(c1 ? v[1] : v[3]);
  const float a0 = c1 ? x0 : v[0], a1 = c1 ? x1 : v[1];  // rows 2 c1, 2 c1 + 1 of column c%2
  const float a2 = c1 ? v[2] : x0, a3 = c1 ? v[3] : x1;  // the same rows of column c%2 + 2
  const float y0 = quad_swap1f(c0 ? a0 : a1);
  const float y1 = quad_swap1f(c0 ? a2 : a3);
  v[0] = c0 ? y0 : a0;
  v[1] = c0 ? a1 : y0;
  v[2] = c0 ? y1 : a2;
  v[3] = c0 ? a3 : y1;
}

// The same transpose for values bound for bf16: rounded (to nearest even)
// and packed first, so the exchanges move half as many words; the second
// exchange splices 16-bit halves with v_perm_b32 (selector bytes 0-3 pick
// bytes of the second operand, 4-7 of the first). Returns row c, columns
// 0..3, as four bf16.
__device__ __forceinline__ u32x2 quad_transpose_bf16(const float (&v)[4], int lane) {
  const bool c1 = (lane & 2) != 0, c0 = (lane & 1) != 0;
  const uint32_t p0 = pack_bf16x2(v[0], v[1]);  // rows 0 (low half), 1 of column c
  const uint32_t p1 = pack_bf16x2(v[2], v[3]);  // rows 2, 3
  const uint32_t x = quad_swap2(c1 ? p0 : p1);
  const uint32_t a0 = c1 ? x : p0;  // rows 2 c1, 2 c1 + 1 of column c%2
  const uint32_t a1 = c1 ? p1 : x;  // the same rows of column c%2 + 2
  const uint32_t y0 = quad_swap1(a0), y1 = quad_swap1(a1);
  const uint32_t sel = c0 ? 0x03020706u : 0x05040100u;  // high halves / low halves, in column order
  return u32x2{__builtin_amdgcn_perm(y0, a0, sel), __builtin_amdgcn_perm(y1, a1, sel)};
}

// Exchange with lane l ^ 4: a DPP row shift left by 4 writes the lanes with
// bit 2 clear (banks 0 and 2 of each 16-lane row), a shift right by 4 the
// others (banks 1 and 3).
__device__ __forceinline__ uint32_t swap4(uint32_t v) {
  const int a = __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x104, 0xF, 0x5, false);
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(a, static_cast<int>(v), 0x114, 0xF, 0xA, false));
}
// Two quad-transposed bf16 results of column blocks 2jp (t0) and 2jp + 1
// (t1), same row, into eight consecutive columns per lane: lanes with bit 2
// clear take columns 8m .. 8m + 7 (m = lane%32 / 8) of block 2jp, the others
// the same columns of block 2jp + 1. A store of the result covers eight rows
// (four per wavefront half) x 64 columns.
__device__ __forceinline__ u32x4 pair_cols8(u32x2 t0, u32x2 t1, int lane) {
  const bool hi = (lane & 4) != 0;
  const u32x2 send = hi ? t0 : t1;
  const uint32_t r0 = swap4(send.x), r1 = swap4(send.y);
  return hi ? u32x4{r0, r1, t1.x, t1.y} : u32x4{t0.x, t0.y, r0, r1};
}

// The same for fp32 values: eight consecutive columns of one row in o.
__device__ __forceinline__ void pair_cols8(const float (&t0)[4], const float (&t1)[4], int lane, float (&o)[8]) {
  const bool hi = (lane & 4) != 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float r = __uint_as_float(swap4(__float_as_uint(hi ? t0[q] : t1[q])));
    o[q] = hi ? r : t0[q];
    o[q + 4] = hi ? t1[q] : r;
  }
}

// Exclusive prefix over experts of v (expert tid*4 + j in v[j]) into
// out[0..E], out[E] the total; a block of NT threads, `part` NT ints of LDS.
__device__ __forceinline__ void expert_scan(const int (&v)[4], int* out, int* part, int E, int tid) {
  const int sum = v[0] + v[1] + v[2] + v[3];
  part[tid] = sum;
  __syncthreads();
  for (int o = 1; o < NT; o <<= 1) {
    const int x = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int run = part[tid] - sum;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * 4 + j;
    if (e < E) out[e] = run;
    run += v[j];
  }
  if (tid == NT - 1) out[E] = part[NT - 1];
  __syncthreads();
}

// Split-K plan of the weight gradients. Their reduction runs over an
// expert's rows, a ragged count; an expert far longer than a workgroup's
// share of the launch would keep one CU busy long after the others, so it is
// cut into chunks of about equal length, each a tile of its own:
//   cap       = max(kMinChunkSteps, ceil(W / (2 * grid)))   W = tiles per expert * sum of k-steps
//   chunks(e) = ceil(steps(e) / cap)                         (1 while steps(e) <= cap)
// Chunk 0 writes the gradient; later chunks write fp32 partial tiles to the
// workspace, which a second kernel adds in chunk order (no atomics: the
// result does not depend on timing). Fewer than W / cap <= 2 * grid partial
// tiles exist at any shape.
constexpr int kMinChunkSteps = 64;
__device__ __forceinline__ int split_cap(int work, int grid) {
  return max(kMinChunkSteps, (work + 2 * grid - 1) / (2 * grid));
}
__device__ __forceinline__ int split_chunks(int steps, int cap) { return steps > cap ? (steps + cap - 1) / cap : 1; }
__device__ __forceinline__ int split_len(int steps, int chunks) { return (steps + chunks - 1) / chunks; }

// FUSED (the gather and the routing weights fused into the GEMMs, compiled
// separately so that the plain kernels carry none of it): GATEUP reads its A
// rows through P.row_token and may skip storing G and U; WGRAD_GATEUP reads
// its B k-rows (x) through P.row_token; DOWN scales its output rows by
// P.row_weight.
// The workgroup's LDS. The stages are separate objects: with the stage of
// every access known at compile time, the compiler sees that loads landing in
// one stage do not alias reads of another and does not wait for them before
// reading.
struct Smem {
  bf16_t (&lds0)[STAGE];
  bf16_t (&lds1)[STAGE];
  bf16_t (&lds2)[STAGE];
  bf16_t (&lds3)[STAGE];
  int (&tstart)[1025];  // grouped-M: first m-tile of each expert; grouped-K: first tile
  int (&pstart)[1025];  // grouped-K: first partial tile of each expert
  int (&wstart)[1025];  // grouped-K: work (k-steps) before each expert's tiles
  int (&part)[NT];
  int (&eoff)[1025];    // offsets[0..E]: read at every tile start, from LDS rather than
                        // through a vector load whose wait would drain the prefetches
};
#define MOE_GEMM_SMEM                                          \
  __shared__ __attribute__((aligned(16))) bf16_t lds0[STAGE]; \
  __shared__ __attribute__((aligned(16))) bf16_t lds1[STAGE]; \
  __shared__ __attribute__((aligned(16))) bf16_t lds2[STAGE]; \
  __shared__ __attribute__((aligned(16))) bf16_t lds3[STAGE]; \
  __shared__ int tstart[1025];                                 \
  __shared__ int pstart[1025];                                 \
  __shared__ int wstart[1025];                                 \
  __shared__ int part[NT];                                     \
  __shared__ int eoff[1025];                                   \
  const Smem sm{lds0, lds1, lds2, lds3, tstart, pstart, wstart, part, eoff};

// Every tile of one GEMM that workgroup `bid` of `nblk` (a multiple of 8)
// owns, start to finish: on return every load and store this workgroup
// issued has completed and its waves are past a barrier.
template <int MODE, bool FUSED, bool F8 = false, bool AW = false, bool F4 = false, bool KX = false>
__device__ __forceinline__ void gemm_tiles(const Params& P, const int bid, const int nblk, const Smem& sm) {
  static_assert(!F8 || (FUSED && (MODE == GATEUP || MODE == DOWN)), "fp8: the inference forward's two GEMMs");
  static_assert(!F4 || F8, "MXFP4 weights: with fp8 activations");
  static_assert(!KX || (!F8 && !AW && !grouped_k(MODE) && (!FUSED || MODE == GATEUP || MODE == DGRAD_DOWN)),
                "extended K: the bf16 forward and data-gradient GEMMs (gate/up and down dgrad also with gathered rows)");
  static_assert(!AW || (MODE == GATEUP && !F8), "a_w: the gate/up GEMM of the training step");
  // Element size in bytes, elements per k-step (64 bytes of a k-major row
  // either way) and per 16-byte chunk.
  constexpr int ESZ = F8 ? 1 : 2;
  constexpr int KS = F8 ? 64 : BK;
  constexpr int CK = 16 / ESZ;
  bf16_t (&lds0)[STAGE] = sm.lds0;
  bf16_t (&lds1)[STAGE] = sm.lds1;
  bf16_t (&lds2)[STAGE] = sm.lds2;
  bf16_t (&lds3)[STAGE] = sm.lds3;
  int (&tstart)[1025] = sm.tstart;
  int (&pstart)[1025] = sm.pstart;
  int (&wstart)[1025] = sm.wstart;
  int (&part)[NT] = sm.part;
  int (&eoff)[1025] = sm.eoff;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lane_id = lane;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  const int wm = wave >> 1, wn = wave & 1;
  const int H = P.H, E = P.E, I = P.I;

  for (int x = tid; x <= E; x += NT) eoff[x] = P.offsets[x];  // visible after the scans' barriers

  // ---- tile list -----------------------------------------------------------
  int ntn, total;
  int tpe = 0, kcap = 0;
  if constexpr (!grouped_k(MODE)) {
    // tstart[e] = sum over e' < e of ceil(count[e'] / BM): 4 experts per thread.
    int loc[4];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid * 4 + j;
      loc[j] = e < E ? (P.offsets[e + 1] - P.offsets[e] + BM - 1) / BM : 0;
      sum += loc[j];
    }
    part[tid] = sum;
    __syncthreads();
    for (int o = 1; o < NT; o <<= 1) {
      const int v = tid >= o ? part[tid - o] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    int run = part[tid] - sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid * 4 + j;
      if (e < E) tstart[e] = run;
      run += loc[j];
    }
    if (tid == NT - 1) tstart[E] = part[NT - 1];
    __syncthreads();
    int ncols;
    if constexpr (MODE == GATEUP) ncols = I;
    else if constexpr (MODE == DOWN) ncols = H;
    else if constexpr (MODE == DGRAD_DOWN) ncols = I;
    else ncols = H;
    ntn = (ncols + (MODE == GATEUP ? GU_COLS : BN) - 1) / (MODE == GATEUP ? GU_COLS : BN);
    total = tstart[E] * ntn;
  } else {
    // Tiles of expert e: chunks(e) x tpe, chunk-major; the split plan above.
    const int mrows = MODE == WGRAD_DOWN ? H : 2 * I;
    const int ncols = MODE == WGRAD_DOWN ? I : H;
    ntn = (ncols + BN - 1) / BN;
    tpe = ((mrows + BM - 1) / BM) * ntn;
    int st[4], c[4], v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid * 4 + j;
      st[j] = e < E ? (P.offsets[e + 1] - P.offsets[e] + BK - 1) / BK : 0;
    }
    expert_scan(st, wstart, part, E, tid);
    kcap = split_cap(tpe * wstart[E], nblk);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = tid * 4 + j < E ? split_chunks(st[j], kcap) : 0;
      v[j] = c[j] * tpe;
    }
    expert_scan(v, tstart, part, E, tid);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = c[j] > 0 ? (c[j] - 1) * tpe : 0;
    expert_scan(v, pstart, part, E, tid);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = c[j] * tpe * (c[j] > 0 ? max(1, split_len(st[j], c[j])) : 0);
    expert_scan(v, wstart, part, E, tid);
    total = tstart[E];
  }

  // Tile range of this workgroup's XCD: an eighth of the tiles (grouped-M:
  // all tiles cost the same) or of the work (grouped-K: tiles of one expert
  // cost the same, those of different experts do not).
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int nslots = nblk >> 3;
  auto tile_at = [&](int x8) -> int {
    if constexpr (!grouped_k(MODE)) {
      return static_cast<int>((static_cast<int64_t>(total) * x8) / 8);
    } else {
      const int w = static_cast<int>((static_cast<int64_t>(wstart[E]) * x8) / 8);
      if (x8 >= 8) return total;
      int l2 = 0, h2 = E - 1;
      while (l2 < h2) {
        const int mid = (l2 + h2 + 1) >> 1;
        if (wstart[mid] <= w) l2 = mid; else h2 = mid - 1;
      }
      const int tiles = tstart[l2 + 1] - tstart[l2];
      const int wt = (wstart[l2 + 1] - wstart[l2]) / tiles;
      return tstart[l2] + min(tiles, (w - wstart[l2] + wt - 1) / wt);
    }
  };
  const int lo = tile_at(xcd);
  const int hi = tile_at(xcd + 1);

  constexpr bool A_KMAJOR = !grouped_k(MODE);
  constexpr bool B_KMAJOR = b_kcontig(MODE);
  // Rows of a k-major A read through row_token (x for gate/up, dy for the
  // down data gradient): per-lane offsets set at each tile start.
  constexpr bool GATHER_A_ROWS = (MODE == GATEUP || MODE == DGRAD_DOWN) && FUSED;
  // Weight gradients with an operand read through row_token: the k-rows of
  // B (x, gate/up) or of A (dy, down) are gathered, so that operand's load
  // offsets change with every k-step.
  constexpr bool GATHER_B = MODE == WGRAD_GATEUP && FUSED;
  constexpr bool GATHER_A = MODE == WGRAD_DOWN && FUSED;
  constexpr bool GATHER_K = GATHER_A || GATHER_B;

  // ---- tile state ------------------------------------------------------------
  // Everything the operand loads of a tile depend on. A tile's last k-step
  // already loads the next tile's first one, so the state moves on to the
  // next tile before the finished tile's epilogue, which keeps its own copy
  // of the few scalars it needs.
  int lda = 0, ldb = 0, kfixed = 0;
  if constexpr (MODE == GATEUP) { lda = H; kfixed = H / KS; }
  if constexpr (MODE == DOWN) { lda = I; kfixed = I / KS; }
  if constexpr (MODE == DGRAD_DOWN) { lda = H; ldb = I; kfixed = H / BK; }
  if constexpr (MODE == DGRAD_GATEUP) { lda = 2 * I; ldb = H; kfixed = 2 * I / BK; }
  if constexpr (MODE == WGRAD_DOWN) { lda = H; ldb = I; }
  if constexpr (MODE == WGRAD_GATEUP) { lda = 2 * I; ldb = H; }
  const int kmain = kfixed;  // k-steps of the main operands; KX: then P.kx / BK more
  if constexpr (KX) kfixed += P.kx / BK;
  // KX: the adapter column of extension step s (gate/up: within its half).
  auto ext_col = [&](int s) -> int {
    const int k0x = (s - kmain) * BK;
    return MODE == GATEUP && k0x >= P.kxp ? k0x - P.kxp : k0x;
  };

  int e = 0, row0 = 0, mvalid = 0, m0 = 0, n0 = 0, kbeg = 0, kend = 0, ksteps = 0;
  int pidx = -1;  // grouped-K: partial tile of a later chunk, -1 for chunk 0
  int nkbeg = 0;  // GATHER_K: first k-row of this workgroup's next tile
  uint32_t aoff[LOADS / 2], boff[LOADS / 2];
  // MXFP4 B stage: LDS block of this wavefront's load t. Data blocks 0-7
  // (t < 2): gate/up rows 32 b .. are gate for b in {0, 1, 4, 5}, up for
  // {2, 3, 6, 7}; scales in block 8 (gate or down) and 9 (up); the loads
  // that fetch nothing get blocks 10-15 of their own.
  auto f4_slot = [&](int t) -> int {
    if (t < 2) return (wave & 1) * 4 + (wave >> 1) * 2 + t;
    if (t == 2) return MODE == GATEUP ? 8 + (wave >> 1) + 2 * (wave & 1) : 8 + wave;
    return 12 + wave;
  };
  // Chunk swizzle of the 32-byte MXFP4 rows: 8 lanes reading one chunk of
  // 8 consecutive rows hit 32 distinct banks.
  auto sw4 = [](int r) -> int { return (r >> 2) & 1; };
  uint32_t gcol[LOADS / 2];  // GATHER_K: column byte offsets of the gathered operand's loads
  const char* abase_m = reinterpret_cast<const char*>(P.a);  // grouped-M: the tile's first row of A

  // Grouped-K: the first k-row of tile Lx's chunk.
  auto kbeg_of = [&](int Lx) -> int {
    int l2 = 0, h2 = E - 1;
    while (l2 < h2) {
      const int mid = (l2 + h2 + 1) >> 1;
      if (tstart[mid] <= Lx) l2 = mid; else h2 = mid - 1;
    }
    const int ob = eoff[l2], oe = eoff[l2 + 1];
    const int steps = (oe - ob + BK - 1) / BK;
    return ob + (Lx - tstart[l2]) / tpe * split_len(steps, split_chunks(steps, kcap)) * BK;
  };
  auto set_tile = [&](int L) __attribute__((always_inline)) {
    int te, trow0 = 0, tmvalid = 0, tm0 = 0, tn0 = 0, tkbeg = 0, tkend = 0, tpidx = -1;
    if constexpr (!grouped_k(MODE)) {
      int l2 = 0, h2 = E - 1;
      while (l2 < h2) {
        const int mid = (l2 + h2 + 1) >> 1;
        if (tstart[mid] * ntn <= L) l2 = mid; else h2 = mid - 1;
      }
      te = l2;
      const int rem = L - tstart[te] * ntn;
      const int mte = tstart[te + 1] - tstart[te];
      const int nt = rem / mte;
      const int mt = rem - nt * mte;
      // The expert's rows split evenly over its mte tiles (at most BM each):
      // no short last tile that would race ahead of its siblings, fetching
      // the weight slice they share on its own.
      const int64_t cnt = eoff[te + 1] - eoff[te];
      const int r0 = static_cast<int>((mt * cnt) / mte);
      trow0 = eoff[te] + r0;
      tmvalid = static_cast<int>(((mt + 1) * cnt) / mte) - r0;
      tn0 = nt * (MODE == GATEUP ? GU_COLS : BN);
    } else {
      int l2 = 0, h2 = E - 1;
      while (l2 < h2) {
        const int mid = (l2 + h2 + 1) >> 1;
        if (tstart[mid] <= L) l2 = mid; else h2 = mid - 1;
      }
      te = l2;
      const int rem = L - tstart[te];
      const int chunk = rem / tpe;
      const int t = rem - chunk * tpe;
      const int mt = t / ntn;
      const int nt = t - mt * ntn;
      tm0 = mt * BM;
      tn0 = nt * BN;
      const int ob = eoff[te], oe = eoff[te + 1];
      const int steps = (oe - ob + BK - 1) / BK;
      const int len = split_len(steps, split_chunks(steps, kcap)) * BK;
      tkbeg = ob + chunk * len;
      tkend = min(oe, tkbeg + len);
      tpidx = chunk > 0 ? pstart[te] + (chunk - 1) * tpe + t : -1;
    }
    // The decode is the same on every lane; say so, so that the operand
    // bases live in scalar registers and the loads use the scalar-base form.
    e = __builtin_amdgcn_readfirstlane(te);
    row0 = __builtin_amdgcn_readfirstlane(trow0);
    mvalid = __builtin_amdgcn_readfirstlane(tmvalid);
    m0 = __builtin_amdgcn_readfirstlane(tm0);
    n0 = __builtin_amdgcn_readfirstlane(tn0);
    kbeg = __builtin_amdgcn_readfirstlane(tkbeg);
    kend = __builtin_amdgcn_readfirstlane(tkend);
    pidx = __builtin_amdgcn_readfirstlane(tpidx);
    ksteps = grouped_k(MODE) ? (kend - kbeg + BK - 1) / BK : kfixed;
    if constexpr (GATHER_K)  // the row tokens run two steps ahead, into the next tile
      nkbeg = __builtin_amdgcn_readfirstlane(L + nslots < hi ? kbeg_of(L + nslots) : 0);
  };
  // Per-lane load offsets of the current tile (vector registers; recomputed
  // rather than kept alive across an epilogue).
  auto set_offsets = [&](auto ext, int kk = 0) __attribute__((always_inline)) {
    // ext (KX): the extension's offsets: A's rows of length P.kx; k-major
    // B's rows are the adapters' (length P.kxr), at their column kk of this
    // step, and a lane whose 8 columns lie past the rank loads nothing.
    constexpr bool EXT = decltype(ext)::value;
    // An opaque copy of the lane index keeps the lane-only parts of these
    // offsets from being hoisted out of the tile loop (and spilled).
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    // Per-lane byte offsets of this wavefront's 4 + 4 load instructions,
    // relative to the operand's base at the current k-step; instruction t
    // fills LDS block wave*4 + t (1 KiB) of each operand stage. Rows and
    // columns past the operand's end are clamped to its last one, or (A rows
    // of a grouped-M tile) fall outside the buffer range and read as zeros;
    // either way their products land in rows or columns that are never
    // stored. k-major: LDS row r = 16 (wave*4 + t) + lane/4, chunk lane%4
    // (swizzled). mn-major: k-row 2 (wave*4 + t) + lane/32, chunk lane%32
    // (swizzled).
#pragma unroll
    for (int t = 0; t < LOADS / 2; ++t) {
      const int blk = wave * (LOADS / 2) + t;
      if constexpr (A_KMAJOR) {
        const int r = blk * 16 + (lane >> 2);
        const int c = (lane & 3) ^ swk(r);
        if (GATHER_A_ROWS && !EXT)  // row of x or dy; rows >= mvalid read zeros (the extension's rows are sorted)
          aoff[t] = r < mvalid ? ESZ * (static_cast<uint32_t>(P.row_token[row0 + r]) * H + c * CK) : kNoWrite;
        else
          aoff[t] = ESZ * (r * (EXT ? P.kx : lda) + c * CK);  // rows >= mvalid: outside the range, read as zeros
      } else {
        const int k = blk * 2 + (lane >> 5);
        const int c = (lane & 31) ^ swt(k);
        const int mrows = MODE == WGRAD_DOWN ? H : 2 * I;
        if constexpr (GATHER_A) gcol[t] = 2u * min(m0 + c * 8, mrows - 8);  // row part: gather_off
        else aoff[t] = 2u * (k * lda + min(m0 + c * 8, mrows - 8));
      }
      if constexpr (F4) {
        // MXFP4 B: a k-step is 32 bytes of a weight row, two 16-byte chunks
        // swapped on rows with bit 2 set (sw4). Instructions 0 and 1 of a
        // wavefront fill data block f4_slot (32 rows each: lane l, row
        // 32 slot + l/2); in gate/up, wavefronts 0 and 1 hold the gate rows,
        // 2 and 3 the up rows, so that each reads one weight. Instruction 2
        // of wavefront 0 (and 2 for up) loads the step's two block scales of
        // the 256 rows; the rest load nothing (see rsrc_b4).
        const int K2 = MODE == GATEUP ? H / 2 : I / 2;  // bytes per weight row
        if (t < 2) {
          const int r = f4_slot(t) * 32 + (lane >> 1);
          const int c = (lane & 1) ^ sw4(r);
          int idx;
          if constexpr (MODE == GATEUP) idx = min(n0 + (r >> 7) * 64 + (r & 63), I - 1);
          else idx = min(n0 + r, H - 1);
          boff[t] = static_cast<uint32_t>(idx * K2 + c * 16);
        } else if (t == 2 && (MODE == GATEUP ? (wave & 1) == 0 : wave == 0)) {
          if constexpr (MODE == GATEUP)  // lanes 0-15: block lane/8, half (lane/4)%2, 16 rows 16 (lane%4) ..
            boff[t] = lane < 16 ? static_cast<uint32_t>((lane >> 3) * I + n0 + ((lane >> 2) & 1) * 64 + 16 * (lane & 3))
                                : kNoWrite;
          else  // lanes 0-31: block lane/16, 16 rows 16 (lane%16) ..
            boff[t] = lane < 32 ? static_cast<uint32_t>((lane >> 4) * H + n0 + 16 * (lane & 15)) : kNoWrite;
        } else {
          boff[t] = kNoWrite;
        }
      } else if constexpr (MODE == GATEUP) {
        // LDS row r: wavefront column half r / 128 and 32-column block
        // j = (r % 128) / 32 of it (j < 2: gate, j >= 2: up, same indices).
        // A wavefront's 64 rows are all gate (even waves) or all up (odd).
        const int r = blk * 16 + (lane >> 2);
        const int c = (lane & 3) ^ swk(r);
        const int j = (r & 127) >> 5;
        const int idx = min(n0 + (r >> 7) * 64 + (j & 1) * 32 + (r & 31), I - 1);
        if constexpr (EXT) boff[t] = c * CK + kk < P.kxr ? ESZ * (idx * P.kxr + c * CK) : kNoWrite;
        else boff[t] = ESZ * (idx * H + c * CK);
      } else if constexpr (MODE == DOWN) {
        const int r = blk * 16 + (lane >> 2);
        const int c = (lane & 3) ^ swk(r);
        if constexpr (EXT) boff[t] = c * CK + kk < P.kxr ? ESZ * (min(n0 + r, H - 1) * P.kxr + c * CK) : kNoWrite;
        else boff[t] = ESZ * (min(n0 + r, H - 1) * I + c * CK);
      } else {
        const int k = blk * 2 + (lane >> 5);
        const int c = (lane & 31) ^ swt(k);
        const int ncols = (MODE == DGRAD_DOWN || MODE == WGRAD_DOWN) ? I : H;
        if constexpr (GATHER_B) gcol[t] = 2u * min(n0 + c * 8, ncols - 8);  // row part: gather_off
        else boff[t] = 2u * (k * ldb + min(n0 + c * 8, ncols - 8));
      }
    }
    if constexpr (!EXT) abase_m = reinterpret_cast<const char*>(P.a) + static_cast<int64_t>(row0) * lda * ESZ;
  };
  // No next tile: every load of the chained step reads an empty range.
  auto clear_tile = [&]() {
    ksteps = 0;
    kend = kbeg;
  };
  auto set_tile_and_offsets = [&](int L) __attribute__((always_inline)) {
    set_tile(L);
    set_offsets(std::false_type{});
  };


  // Buffer resources of k-step s (num_records 0 past the last step).
  auto rsrc_a = [&](int s) -> rsrc_t {
    if constexpr (KX) {
      if (s >= kmain) {  // the extension: rows of length kx, from the tile's first row
        const int k0x = (s - kmain) * BK;
        return make_rsrc(reinterpret_cast<const char*>(P.ax) + (static_cast<int64_t>(row0) * P.kx + k0x) * ESZ,
                         s < ksteps ? ESZ * (mvalid * P.kx - k0x) : 0);
      }
    }
    const int k0 = s * KS;
    if constexpr (A_KMAJOR) {
      if (GATHER_A_ROWS)
        return make_rsrc(reinterpret_cast<const char*>(P.a) + k0 * ESZ, s < ksteps ? ESZ * (P.T * H - k0) : 0);
      return make_rsrc(abase_m + k0 * ESZ, s < ksteps ? ESZ * (mvalid * lda - k0) : 0);
    } else {
      const int left = kend - kbeg - k0;
      if constexpr (GATHER_A) return make_rsrc(P.a, left > 0 ? 2 * P.T * H : 0);
      return make_rsrc(P.a + static_cast<int64_t>(kbeg + k0) * lda, left > 0 ? 2 * left * lda : 0);
    }
  };
  auto rsrc_b = [&](int s) -> rsrc_t {
    if constexpr (KX) {
      if (s >= kmain) {
        // Step s's rank columns (or k-rows) kk of one adapter: gate/up's
        // first kxp steps are the gate adapter's, the next kxp the up one's
        // (in the forward, a wavefront of the other half reads nothing).
        const int k0x = (s - kmain) * BK;
        const bool second = (MODE == GATEUP || MODE == DGRAD_GATEUP) && k0x >= P.kxp;
        const int kk = second ? k0x - P.kxp : k0x;
        const bool live = s < ksteps && kk < P.kxr;
        const int64_t r = P.kxr;
        if constexpr (MODE == GATEUP) {
          const bool mine = ((wave & 1) != 0) == second;  // odd wavefronts: the up columns
          return make_rsrc((second ? P.bx1 : P.bx0) + (static_cast<int64_t>(e) * I * r + kk),
                           live && mine ? ESZ * (I * P.kxr - kk) : 0);
        } else if constexpr (MODE == DOWN) {
          return make_rsrc(P.bx0 + (static_cast<int64_t>(e) * H * r + kk), live ? ESZ * (H * P.kxr - kk) : 0);
        } else if constexpr (MODE == DGRAD_DOWN) {  // k-rows past the rank: outside the range, zeros
          return make_rsrc(P.bx0 + (static_cast<int64_t>(e) * r + kk) * I, live ? 2 * (P.kxr - kk) * I : 0);
        } else {
          return make_rsrc((second ? P.bx1 : P.bx0) + (static_cast<int64_t>(e) * r + kk) * H,
                           live ? 2 * (P.kxr - kk) * H : 0);
        }
      }
    }
    const int k0 = s * KS;
    const bool live = s < ksteps;
    if constexpr (MODE == GATEUP) {
      const char* w = reinterpret_cast<const char*>((wave & 1) ? P.b1 : P.b0) + (static_cast<int64_t>(e) * I * H + k0) * ESZ;
      return make_rsrc(w, live ? ESZ * (I * H - k0) : 0);
    } else if constexpr (MODE == DOWN) {
      return make_rsrc(reinterpret_cast<const char*>(P.b0) + (static_cast<int64_t>(e) * H * I + k0) * ESZ,
                       live ? ESZ * (H * I - k0) : 0);
    } else if constexpr (MODE == DGRAD_DOWN) {
      return make_rsrc(P.b0 + static_cast<int64_t>(e) * H * I + static_cast<int64_t>(k0) * I,
                       live ? 2 * (H - k0) * I : 0);
    } else if constexpr (MODE == DGRAD_GATEUP) {
      const bool up = k0 >= I;
      const int kk0 = up ? k0 - I : k0;
      return make_rsrc((up ? P.b1 : P.b0) + static_cast<int64_t>(e) * I * H + static_cast<int64_t>(kk0) * H,
                       live ? 2 * (I - kk0) * H : 0);
    } else {
      const int left = kend - kbeg - k0;
      if constexpr (GATHER_B) return make_rsrc(P.b0, left > 0 ? 2 * P.T * H : 0);
      return make_rsrc(P.b0 + static_cast<int64_t>(kbeg + k0) * ldb, left > 0 ? 2 * left * ldb : 0);
    }
  };

  // GATHER_K: the row tokens of the gathered operand's k-rows. Instruction t
  // of a wavefront's A or B loads covers k-rows 8 wave + 2t (lanes 0-31) and
  // 8 wave + 2t + 1 (lanes 32-63) of its step; lane l fetches the token of k-row
  // 8 wave + 2 (l % 4) + l / 32, so that lanes t and 32 + t hold the two rows
  // of instruction t. Step q of the current tile, or (q past the tile's
  // padded step count) step q - that count of the next one. Reads past the
  // end of row_token return 0; such rows are never used.
  const rsrc_t rtok = make_rsrc(P.row_token, GATHER_K ? 4 * P.M : 0);
  auto load_tok = [&](int q) -> uint32_t {
    const int nst = max(NSTAGE, (ksteps + NSTAGE - 1) / NSTAGE * NSTAGE);
    const bool nxt = q >= nst;
    int lane = lane_id;  // opaque copy: the lane term is recomputed here, not kept alive (and spilled)
    asm volatile("" : "+v"(lane));
    const int row = (nxt ? nkbeg : kbeg) + (nxt ? q - nst : q) * BK + wave * 8 + 2 * (lane & 3) + (lane >> 5);
    return __builtin_amdgcn_raw_buffer_load_b32(rtok, 4u * static_cast<uint32_t>(row), 0, 0);
  };
  // The gathered operand's byte offsets for step sn of the current tile
  // from its tokens: row token * 2H (x and dy rows are H long) plus the
  // column part; k-rows past the chunk's end get an offset outside the range
  // (zeros).
  auto gather_off = [&](uint32_t tok, int sn) __attribute__((always_inline)) {
    const int left = kend - kbeg - sn * BK - wave * 8;
    const bool hi32 = lane_id >= 32;
#pragma unroll
    for (int t = 0; t < LOADS / 2; ++t) {
      const uint32_t t0 = __builtin_amdgcn_readlane(tok, t);
      const uint32_t t1 = __builtin_amdgcn_readlane(tok, 32 + t);
      const uint32_t o0 = 2 * t < left ? t0 * (2u * H) : kNoWrite;
      const uint32_t o1 = 2 * t + 1 < left ? t1 * (2u * H) : kNoWrite;
      const uint32_t o = (hi32 ? o1 : o0) + gcol[t];
      if constexpr (GATHER_A) aoff[t] = o;
      else boff[t] = o;
    }
  };
  // Tokens of steps sn and sn + 1 at the start of the k-step that loads sn.
  uint32_t tkA = 0, tkB = 0;

  // Load instruction v of a k-step's 8, for step sn into the stage at L:
  // even v an A block, odd v a B block (block v/2 of this wavefront's 4).
  auto vmem = [&](int v, const rsrc_t& ra, const rsrc_t& rb, bf16_t* L) __attribute__((always_inline)) {
    const int t = v >> 1;
    if ((v & 1) == 0) buf_to_lds16(ra, aoff[t], L + (wave * (LOADS / 2) + t) * 512);
    else buf_to_lds16(rb, boff[t], L + STAGE_A + (wave * (LOADS / 2) + t) * 512);
  };
  // MXFP4 B (F4), k-step s: the wavefront's data resource (gate or down
  // weight, or up for wavefronts 2 and 3 of gate/up) and scale resource
  // (the step's two E8M0 blocks of every row, scales stored [E][K/32][N]:
  // one block's scales of consecutive rows are contiguous).
  auto rsrc_b4 = [&](int s) -> rsrc_t {
    const int k0 = s * KS;
    const bool live = s < ksteps;
    if constexpr (MODE == GATEUP) {
      const char* w = reinterpret_cast<const char*>((wave >> 1) ? P.b1 : P.b0) + (static_cast<int64_t>(e) * I * H + k0) / 2;
      return make_rsrc(w, live ? (I * H - k0) / 2 : 0);
    } else {
      return make_rsrc(reinterpret_cast<const char*>(P.b0) + (static_cast<int64_t>(e) * H * I + k0) / 2,
                       live ? (H * I - k0) / 2 : 0);
    }
  };
  auto rsrc_s4 = [&](int s) -> rsrc_t {
    const bool live = s < ksteps;
    if constexpr (MODE == GATEUP) {
      const uint8_t* sc = ((wave >> 1) ? P.sb1 : P.sb0) + (static_cast<int64_t>(e) * (H / 32) + 2 * s) * I;
      return make_rsrc(sc, live ? 2 * I : 0);
    } else {
      return make_rsrc(P.sb0 + (static_cast<int64_t>(e) * (I / 32) + 2 * s) * H, live ? 2 * H : 0);
    }
  };
  auto vmem4 = [&](int v, const rsrc_t& ra, const rsrc_t& rd, const rsrc_t& rs, bf16_t* L)
                   __attribute__((always_inline)) {
    const int t = v >> 1;
    if ((v & 1) == 0) buf_to_lds16(ra, aoff[t], L + (wave * (LOADS / 2) + t) * 512);
    else buf_to_lds16(t < 2 ? rd : rs, boff[t], L + STAGE_A + f4_slot(t) * 512);
  };
  // All 8 at once (the first steps of a workgroup's first tile).
  auto issue = [&](int s, bf16_t* L) __attribute__((always_inline)) {
    if constexpr (KX) {
      if (s >= kmain) set_offsets(std::true_type{}, ext_col(s));
    }
    const rsrc_t ra = rsrc_a(s);
    if constexpr (F4) {
      const rsrc_t rd = rsrc_b4(s), rs = rsrc_s4(s);
#pragma unroll
      for (int v = 0; v < LOADS; ++v) vmem4(v, ra, rd, rs, L);
    } else {
      const rsrc_t rb = rsrc_b(s);
#pragma unroll
      for (int v = 0; v < LOADS; ++v) vmem(v, ra, rb, L);
    }
  };

  // Operand fragments of k-slice kk (16 k; two per step) for 32-row block
  // i, as byte offsets inside a stage. k-major (ds_read_b128, lane: row
  // i*32 + lane%32, chunk 2 kk + lane/32): the chunk XOR makes slice kk the
  // slice-0 offset XOR 32 kk. mn-major (two ds_read_b64_tr_b16, lane: k-row
  // 8 (lane/32) + (lane%16)/4, columns 4 (lane%4) .. + 3 of the block's
  // 16-column half (lane/16)%2): slice kk adds 16 rows = 8 KiB, the second
  // read 4 rows = 2 KiB.
  int aof[FM], bof[FN];
  // Computed at the start of every tile from an opaque copy of the lane
  // index: alive through the k-loop only, not through the epilogue.
  auto set_frag_offsets = [&]() __attribute__((always_inline)) {
  int lane = lane_id;
  asm volatile("" : "+v"(lane));
  const int hi32 = lane >> 5;
  const int g16 = lane >> 4, i16 = lane & 15;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if constexpr (A_KMAJOR) {
      const int r = wm * WTM + i * 32 + (lane & 31);
      aof[i] = r * (BK * 2) + ((hi32 ^ swk(r)) << 4);
    } else {
      const int k = 8 * (g16 >> 1) + (i16 >> 2);
      const int col = wm * WTM + i * 32 + 16 * (g16 & 1) + 4 * (i16 & 3);
      aof[i] = k * 512 + (((col >> 3) ^ swt(k)) << 4) + ((col & 7) << 1);
    }
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    if constexpr (B_KMAJOR) {
      const int r = wn * WTN + j * 32 + (lane & 31);
      bof[j] = r * (BK * 2) + ((hi32 ^ swk(r)) << 4);
    } else {
      const int k = 8 * (g16 >> 1) + (i16 >> 2);
      const int col = wn * WTN + j * 32 + 16 * (g16 & 1) + 4 * (i16 & 3);
      bof[j] = k * 512 + (((col >> 3) ^ swt(k)) << 4) + ((col & 7) << 1);
    }
  }
  };
  auto frag = [&](const bf16_t* S, int off, int kk, bool kmajor) -> bf16x8 {
    const char* base = reinterpret_cast<const char*>(S);
    if (kmajor) return *reinterpret_cast<const bf16x8*>(base + (off ^ (kk * 32)));
    const char* p = base + off + kk * 8192;
    const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
    const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 2048));
    const v4i16 both[2] = {lo4, hi4};
    return __builtin_bit_cast(bf16x8, both);
  };

  f32x16 acc[FM][FN];
  bf16x8 fa0[FM], fb0[FN];  // slice 0 of the step about to run, read during the step before

  // Fragments of k-slice kk of the stage at S (A blocks with valid rows only).
  auto read_slice = [&](auto nbc, const bf16_t* S, int kk, bf16x8 (&fa)[FM], bf16x8 (&fb)[FN])
                        __attribute__((always_inline)) {
    constexpr int nbm = decltype(nbc)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      if (i < nbm) fa[i] = frag(S, aof[i], kk, A_KMAJOR);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      if (nbm > 0) fb[j] = frag(S + STAGE_A, bof[j], kk, B_KMAJOR);
  };
  // The 16 MFMAs of one slice in four groups (row block i); load v0 + i of
  // step sn follows group i, so that the wavefront never stalls on a full
  // address queue with matrix work waiting behind it. The first slice of a
  // tile (zc) starts from a zero accumulator instead of clearing it first.
  auto mfma_slice = [&](auto nbc, auto zc, const bf16x8 (&fa)[FM], const bf16x8 (&fb)[FN], int v0,
                        const rsrc_t& ra, const rsrc_t& rb, bf16_t* Ln) __attribute__((always_inline)) {
    constexpr int nbm = decltype(nbc)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i < nbm) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (decltype(zc)::value)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], f32x16{}, 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
      } else if constexpr (decltype(zc)::value) {
        // Blocks without valid rows are never stored; defined all the same,
        // so that no value of the previous tile stays alive through this one.
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
      }
      __builtin_amdgcn_sched_barrier(0);
      vmem(v0 + i, ra, rb, Ln);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One k-step (32 k) on the stage at Ac, with loads of step sn (three
  // ahead) going into the stage at Ln:
  //   slice 0: MFMAs (fragments already in registers), slice 1's fragment
  //            reads, loads 0-3;
  //   middle:  this wavefront's loads of the next step have landed (all but
  //            the 12 newest: the step after that and this step's first
  //            half) and its fragment reads are done; then the barrier
  //            makes both true for every wavefront, which also frees the
  //            stage read two steps ago for the loads issued from here on;
  //   slice 1: MFMAs, the next step's slice-0 fragments from An, loads 4-7.
  // Scheduling fences keep every group where it is written. A tile's last
  // step (last = true) has no middle and reads nothing ahead: the wait for
  // the next tile's first steps comes after the epilogue.
  auto kstep = [&](auto nbc, auto first, const bf16_t* Ac, const bf16_t* An, int sn, bf16_t* Ln, bool last)
                   __attribute__((always_inline)) {
    if constexpr (GATHER_K) {
      // Step sn's B offsets from tokens loaded two k-steps ago (their wait
      // covers only loads the pipeline has already waited for), then the
      // tokens of step sn + 2, ahead of this step's operand loads.
      gather_off(tkA, sn);
      const uint32_t tn = load_tok(sn + 2);
      tkA = tkB;
      tkB = tn;
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (KX) {  // the extension's steps: its offsets (a tile's last steps, or the next tile's first)
      if (sn >= kmain) set_offsets(std::true_type{}, ext_col(sn));
    }
    const rsrc_t ra = rsrc_a(sn);
    const rsrc_t rb = rsrc_b(sn);
    bf16x8 fa1[FM], fb1[FN];
    __builtin_amdgcn_sched_barrier(0);
    read_slice(nbc, Ac, 1, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_slice(nbc, first, fa0, fb0, 0, ra, rb, Ln);
    if (!last) {
      // GATHER_K: two token loads more among the newest.
      __builtin_amdgcn_s_waitcnt(GATHER_K ? kWaitVm14 : kWaitVm12);
      step_barrier();
      read_slice(nbc, An, 0, fa0, fb0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mfma_slice(nbc, std::false_type{}, fa1, fb1, LOADS / 2, ra, rb, Ln);
  };

  // ---- fp8 k-step -------------------------------------------------------------
  // v_mfma_scale_f32_32x32x64_f8f6f4: one instruction covers a whole 64-byte
  // stage row (64 k). Lane l of an operand holds 32 bytes of row l % 32:
  // stage chunks 2 (l / 32) and 2 (l / 32) + 1 for both A and B, so lanes
  // of the same half multiply the same k (the hardware pairs an A lane's byte
  // j with the B lane's byte j of the same half). The scale operands are the
  // rows' and columns' E8M0 bytes, replicated in every byte and in both
  // halves, so that the instruction applies 2^(Xa + Xb) to every product
  // whichever byte and lane it reads them from.
  //
  // With MXFP4 B (F4) the pairing is by k: B lane l holds the 32 E2M1
  // values (16 bytes, even k in the low nibble) of row l % 32 for k 32 (l /
  // 32) .. + 31, i.e. one 32-element scale block, scaled by the lane's
  // scale byte; an fp8 A lane holds k 16 (l / 32) .. + 15 in its first 16
  // bytes and k 32 + 16 (l / 32) .. + 15 in the other 16 (stage chunks l/32
  // and l/32 + 2). Both were read off in-bounds probes of the instruction.
  i32x8 fa8[FM], fb8[FN];
  int sca[FM], scb[FN];
  int aof8[FM], bof8[FN], sof4[FN];
  auto set_frag_offsets8 = [&]() __attribute__((always_inline)) {
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int h = lane >> 5, h2 = 2 * h;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WTM + i * 32 + (lane & 31);
      aof8[i] = r * 64 + ((swk(r) ^ (F4 ? h : h2)) << 4);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = wn * WTN + j * 32 + (lane & 31);
      if constexpr (F4) {
        bof8[j] = r * 32 + ((h ^ sw4(r)) << 4);
        if constexpr (MODE == GATEUP) {
          const int q = r & 127, hf = r >> 7;
          sof4[j] = (q < 64 ? 8 * 1024 + q : 9 * 1024 + (q - 64)) + h * 128 + hf * 64;
        } else {
          sof4[j] = 8 * 1024 + h * 256 + r;
        }
      } else {
        bof8[j] = r * 64 + ((swk(r) ^ h2) << 4);
      }
    }
  };
  // This tile's scales: rows of A (sorted rows, valid or not: the codes of
  // invalid rows read as zero) and columns of the output (weight rows).
  auto load_scales8 = [&]() __attribute__((always_inline)) {
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = min(wm * WTM + i * 32 + l32, max(mvalid - 1, 0));
      sca[i] = static_cast<int>(P.sa[row0 + r]) * 0x01010101;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (F4) continue;  // block scales: from each k-step's stage
      int v;
      if constexpr (MODE == GATEUP) {  // wavefront columns: 64 gate (j < 2), then 64 up, same indices
        const int idx = min(n0 + wn * 64 + (j & 1) * 32 + l32, I - 1);
        v = (j < 2 ? P.sb0 : P.sb1)[static_cast<int64_t>(e) * I + idx];
      } else {
        const int n = min(n0 + wn * WTN + j * 32 + l32, H - 1);
        v = P.sb0[static_cast<int64_t>(e) * H + n];
      }
      scb[j] = v * 0x01010101;
    }
  };
  auto frag8 = [&](const bf16_t* S, int off) -> i32x8 {
    const char* base = reinterpret_cast<const char*>(S);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + off);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + (off ^ (F4 ? 32 : 16)));
    return i32x8{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                 static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
  };
  // B fragment of column block j from stage S (F4: 16 bytes and the block
  // scale; otherwise as A).
  auto fragb = [&](const bf16_t* S, int j) __attribute__((always_inline)) {
    if constexpr (F4) {
      const char* base = reinterpret_cast<const char*>(S + STAGE_A);
      const u32x4 v = *reinterpret_cast<const u32x4*>(base + bof8[j]);
      fb8[j] = i32x8{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w),
                     0, 0, 0, 0};
      scb[j] = static_cast<int>(*reinterpret_cast<const uint8_t*>(base + sof4[j]));
    } else {
      fb8[j] = frag8(S + STAGE_A, bof8[j]);
    }
  };
  // A tile's first step: row block 0 and every B fragment (the others are
  // read at the start of each step).
  auto read_first8 = [&](auto nbc, const bf16_t* S) __attribute__((always_inline)) {
    constexpr int nbm = decltype(nbc)::value;
    if (nbm > 0) fa8[0] = frag8(S, aof8[0]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      if (nbm > 0) fragb(S, j);
  };
  auto mfma8 = [&](auto zc, int i, int j) __attribute__((always_inline)) {
    if constexpr (decltype(zc)::value)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa8[i], fb8[j], f32x16{}, 0, F4 ? 4 : 0, 0, sca[i],
                                                                 0, scb[j]);
    else
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa8[i], fb8[j], acc[i][j], 0, F4 ? 4 : 0, 0, sca[i],
                                                                 0, scb[j]);
  };
  // One k-step (64 k) on the stage at Ac, loads of step sn into Ln. At entry
  // fa8[0] and fb8[] hold this step's fragments. First the wait for the next
  // step's stage (all but the 8 newest loads, the step after it) and the
  // barrier, which also frees the stage read during the step before for the
  // loads issued from here on; then the other row blocks' fragments of this
  // step. Row blocks run in order, two loads after each block's four MFMAs;
  // block 0's fragment of the next step is read after block 0, and each
  // column's after that column's MFMA of the last valid block.
  auto kstep8 = [&](auto nbc, auto first, const bf16_t* Ac, const bf16_t* An, int sn, bf16_t* Ln, bool last)
                    __attribute__((always_inline)) {
    constexpr int nbm = decltype(nbc)::value;
    const rsrc_t ra = rsrc_a(sn);
    const rsrc_t rb = F4 ? rsrc_b4(sn) : rsrc_b(sn);
    const rsrc_t rs = F4 ? rsrc_s4(sn) : ra;
    if (!last) {
      __builtin_amdgcn_s_waitcnt(kWaitVm8);
      step_barrier();
    }
#pragma unroll
    for (int i = 1; i < FM; ++i)
      if (i < nbm) fa8[i] = frag8(Ac, aof8[i]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i < nbm) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          mfma8(first, i, j);
          if (i == nbm - 1 && !last) fragb(An, j);
        }
      } else if constexpr (decltype(first)::value) {
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (F4) {
        vmem4(2 * i, ra, rb, rs, Ln);
        vmem4(2 * i + 1, ra, rb, rs, Ln);
      } else {
        vmem(2 * i, ra, rb, Ln);
        vmem(2 * i + 1, ra, rb, Ln);
      }
      if (i == 0 && nbm > 0 && !last) fa8[0] = frag8(An, aof8[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- epilogue -------------------------------------------------------------
  // acc[i][j][q] holds wavefront-tile row i*32 + 8*(q/4) + 4*(lane/32) + q%4,
  // column j*32 + lane%32. A quad transpose of each group of four q leaves
  // lane l with row i*32 + 8*(q/4) + 4*(lane/32) + lane%4, columns
  // j*32 + (lane%32)/4*4 .. + 3: four consecutive columns of one row (fp32
  // outputs store these, 8 rows x 128 bytes per store). For bf16 outputs an
  // exchange with lane l ^ 4 (pair_cols8) joins column blocks 2jp and
  // 2jp + 1 into eight columns per lane, so that each 16-byte store covers
  // 8 rows x 128 bytes. Results go out straight from registers through
  // buffer resources whose range ends at the tile's last valid row; columns
  // past the output's end get an offset outside every range. No LDS and no
  // barriers: the next tile's first loads, already in flight, land meanwhile.
  auto epilogue = [&](int te, int trow0, int tmvalid, int tm0, int tn0, int nbm, int tp)
                      __attribute__((always_inline)) {
    // Lane-only terms from an opaque copy of the lane index, so that they
    // are not hoisted out of the tile loop (and spilled).
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int prow = lane & 3;
    if constexpr (MODE == GATEUP) {
      // Wavefront-tile columns 0..63 are gate, 64..127 up, for the same 64
      // intermediate indices: G, U and A = silu(G) U of one element sit in
      // one lane.
      const int64_t base = static_cast<int64_t>(trow0) * I;
      const int bytes = 2 * tmvalid * I;
      const bool store_gu = !FUSED || P.out0 != nullptr;  // the fused forward may keep A only
      const rsrc_t rg = make_rsrc(store_gu ? P.out0 + base : P.out2, store_gu ? bytes : 0);
      const rsrc_t ru = make_rsrc(store_gu ? P.out1 + base : P.out2, store_gu ? bytes : 0);
      const rsrc_t rs = make_rsrc(P.out2 + base, bytes);
      // 16-byte stores (pair_cols8): lane l writes row 8b + 4(l/32) + l%4 of
      // the row block, intermediate indices 32*((l/4)%2) + 8*((l%32)/8) .. + 7
      // of the wavefront's 64.
      const int hrow = 4 * (lane >> 5) + prow;
      const int idx = tn0 + wn * 64 + ((lane >> 2) & 1) * 32 + ((lane & 31) >> 3) * 8;
      // AW: a_w = bf16(row_weight[p] a) as well, from the fp32 a (transposed
      // first, so that each lane holds one row and takes that row's weight).
      const rsrc_t rwr = make_rsrc(P.row_weight + (AW ? trow0 : 0), AW ? 4 * tmvalid : 0);
      const rsrc_t raw = make_rsrc(AW ? P.out3 + base : P.out2, AW ? bytes : 0);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        float rwi[4];
        if constexpr (AW) {
#pragma unroll
          for (int b = 0; b < 4; ++b)
            rwi[b] = i < nbm ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                   rwr, 4u * static_cast<uint32_t>(wm * WTM + i * 32 + 8 * b + hrow), 0, 0))
                             : 0.0f;
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (i >= nbm) continue;  // no valid rows in this block
          const int r = wm * WTM + i * 32 + 8 * b + hrow;
          const uint32_t off = idx < I ? 2u * static_cast<uint32_t>(r * I + idx) : kNoWrite;
          u32x2 gp[2], up[2], ap[2], wp[2];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float g[4], u[4], a[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              g[q] = acc[i][j][4 * b + q];
              u[q] = acc[i][j + 2][4 * b + q];
              a[q] = g[q] * sigmoid_fast(g[q]) * u[q];
            }
            gp[j] = quad_transpose_bf16(g, lane);
            up[j] = quad_transpose_bf16(u, lane);
            if constexpr (AW) {
              quad_transpose(a, lane);  // row 8b + hrow, four columns
              ap[j] = pack_bf16x4v(a);
#pragma unroll
              for (int q = 0; q < 4; ++q) a[q] *= rwi[b];
              wp[j] = pack_bf16x4v(a);
            } else {
              ap[j] = quad_transpose_bf16(a, lane);
            }
          }
          if (store_gu) {
            store_b128(pair_cols8(gp[0], gp[1], lane), rg, off);
            store_b128(pair_cols8(up[0], up[1], lane), ru, off);
          }
          store_b128(pair_cols8(ap[0], ap[1], lane), rs, off);
          if constexpr (AW) store_b128(pair_cols8(wp[0], wp[1], lane), raw, off);
        }
      }
    } else if constexpr (MODE == DOWN || MODE == DGRAD_GATEUP) {
      // 16-byte stores: lane l writes row 8b + 4(l/32) + l%4, columns
      // jp*64 + 32*((l/4)%2) + 8*((l%32)/8) .. + 7 (pair_cols8).
      const rsrc_t ro = make_rsrc(P.out0 + static_cast<int64_t>(trow0) * H, 2 * tmvalid * H);
      const int hrow = 4 * (lane >> 5) + prow;
      const int ncol8 = ((lane >> 2) & 1) * 32 + ((lane & 31) >> 3) * 8;
      // Fused forward (DOWN with row_weight): the weights of this lane's 16
      // rows, read once before the stores.
      constexpr bool weighted = MODE == DOWN && FUSED;
      float rw[FM][4];
      if constexpr (weighted) {
        const rsrc_t rr = make_rsrc(P.row_weight + trow0, 4 * tmvalid);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int b = 0; b < 4; ++b)
            rw[i][b] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rr, 4u * static_cast<uint32_t>(wm * WTM + i * 32 + 8 * b + hrow), 0, 0));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jp = 0; jp < FN / 2; ++jp)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            if (i >= nbm) continue;  // no valid rows in this block
            const int r = wm * WTM + i * 32 + 8 * b + hrow;
            const int n = tn0 + wn * WTN + jp * 64 + ncol8;
            const uint32_t off = n < H ? 2u * static_cast<uint32_t>(r * H + n) : kNoWrite;
            u32x2 t[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              float v[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) v[q] = acc[i][2 * jp + j][4 * b + q];
              if constexpr (weighted) {  // routing weight of this lane's row, applied in fp32 before rounding
                quad_transpose(v, lane);
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] *= rw[i][b];
                t[j] = pack_bf16x4v(v);
              } else {
                t[j] = quad_transpose_bf16(v, lane);
              }
            }
            store_b128(pair_cols8(t[0], t[1], lane), ro, off);
          }
    } else if constexpr (MODE == DGRAD_DOWN) {
      // dA -> dG = dA U silu'(G), dU = dA silu(G), with the saved G and U of
      // the same rows; written side by side as [dG | dU] (row length 2I).
      const int64_t base = static_cast<int64_t>(trow0) * I;
      const rsrc_t rg = make_rsrc(P.g_in + base, 2 * tmvalid * I);
      const rsrc_t ru = make_rsrc(P.u_in + base, 2 * tmvalid * I);
      const rsrc_t ro = make_rsrc(P.out0 + 2 * base, 4 * tmvalid * I);
      // 16-byte lanes (pair_cols8): lane l handles row 8b + 4(l/32) + l%4 of
      // the row block, columns 32*((l/4)%2) + 8*((l%32)/8) .. + 7 of the
      // 64-column pair jp. The saved G and U of a row block (16 loads per
      // lane) are read one row block ahead, so that their latency overlaps
      // the previous block's arithmetic and stores.
      const int hrow = 4 * (lane >> 5) + prow;
      const int ncol8 = ((lane >> 2) & 1) * 32 + ((lane & 31) >> 3) * 8;
      // FUSED (dy read through row_token): dA row p is scaled by
      // row_weight[p] in fp32 first; the weights travel with G and U.
      const rsrc_t rwr = make_rsrc(P.row_weight + (FUSED ? trow0 : 0), FUSED ? 4 * tmvalid : 0);
      typedef u32x4 GU[FN / 2][4];
      float rwb[2][4];
      auto load_gu = [&](int i, GU& gb, GU& ub) __attribute__((always_inline)) {
        if constexpr (FUSED) {
#pragma unroll
          for (int b = 0; b < 4; ++b)
            rwb[i & 1][b] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rwr, 4u * static_cast<uint32_t>(wm * WTM + i * 32 + 8 * b + hrow), 0, 0));
        }
#pragma unroll
        for (int jp = 0; jp < FN / 2; ++jp)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int r = wm * WTM + i * 32 + 8 * b + hrow;
            const int n = tn0 + wn * WTN + jp * 64 + ncol8;
            const uint32_t off = n < I ? 2u * static_cast<uint32_t>(r * I + n) : kNoWrite;
            gb[jp][b] = load_b128(rg, off);
            ub[jp][b] = load_b128(ru, off);
          }
      };
      GU gb[2], ub[2];
      if (nbm > 0) load_gu(0, gb[0], ub[0]);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (i >= nbm) continue;  // no valid rows in this block
        if (i + 1 < FM && i + 1 < nbm) load_gu(i + 1, gb[(i + 1) & 1], ub[(i + 1) & 1]);
        const GU& gc = gb[i & 1];
        const GU& uc = ub[i & 1];
#pragma unroll
        for (int jp = 0; jp < FN / 2; ++jp)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int r = wm * WTM + i * 32 + 8 * b + hrow;
            const int n = tn0 + wn * WTN + jp * 64 + ncol8;
            float da[2][4], d8[8];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
              for (int q = 0; q < 4; ++q) da[j][q] = acc[i][2 * jp + j][4 * b + q];
              quad_transpose(da[j], lane);
            }
            pair_cols8(da[0], da[1], lane, d8);
            if constexpr (FUSED) {
#pragma unroll
              for (int q = 0; q < 8; ++q) d8[q] *= rwb[i & 1][b];
            }
            const u32x4 gw = gc[jp][b], uw = uc[jp][b];
            const uint32_t gwv[4] = {gw.x, gw.y, gw.z, gw.w}, uwv[4] = {uw.x, uw.y, uw.z, uw.w};
            uint32_t dgp[4], dup[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              float dg[2], du[2];
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const float gv = h ? bf16_hi(gwv[w]) : bf16_lo(gwv[w]);
                const float uv = h ? bf16_hi(uwv[w]) : bf16_lo(uwv[w]);
                const float sg = sigmoid_fast(gv);
                dg[h] = d8[2 * w + h] * uv * sg * (1.0f + gv * (1.0f - sg));
                du[h] = d8[2 * w + h] * (gv * sg);
              }
              dgp[w] = pack_bf16x2(dg[0], dg[1]);
              dup[w] = pack_bf16x2(du[0], du[1]);
            }
            const uint32_t off = n < I ? 2u * static_cast<uint32_t>(r * 2 * I + n) : kNoWrite;
            store_b128(u32x4{dgp[0], dgp[1], dgp[2], dgp[3]}, ro, off);
            store_b128(u32x4{dup[0], dup[1], dup[2], dup[3]}, ro, off == kNoWrite ? kNoWrite : off + 2u * I);
          }
      }
    } else {
      // fp32 weight gradient of expert te, rows m0.., columns n0..; a 32-row
      // block lies wholly in dW_gate or wholly in dW_up (I % 64 == 0). A
      // later split-K chunk (tp >= 0) writes its tile to the workspace
      // instead ([256][256], never accumulated).
      const int mrows = MODE == WGRAD_DOWN ? H : 2 * I;
      const int ncols = MODE == WGRAD_DOWN ? I : H;
      const bool to_part = tp >= 0;
      const int ld = to_part ? BN : ncols;  // row length of the destination, floats
      // After the quad transpose lane l holds row 8b + 4(l/32) + l%4 of the
      // 32-row block, columns (l%32)/4*4 .. + 3 of the 32-column block: each
      // store covers 8 rows x 128 bytes. The += form (compiled separately,
      // so the plain form carries none of it) reads the old values first.
      const int hrow = (lane >> 5) * 4 + prow;
      const int lcol = (lane & 31) & ~3;
      auto store_blocks = [&](auto accum) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int mblk = tm0 + wm * WTM + i * 32;
          if (mblk >= mrows) continue;
          float* dst;
          if (to_part) {
            dst = P.part + static_cast<int64_t>(tp) * (BM * BN) + (wm * WTM + i * 32) * BN;
          } else if constexpr (MODE == WGRAD_DOWN) {
            dst = P.dw0 + (static_cast<int64_t>(te) * H + mblk) * I;
          } else {
            dst = mblk < I ? P.dw0 + (static_cast<int64_t>(te) * I + mblk) * H
                           : P.dw1 + (static_cast<int64_t>(te) * I + (mblk - I)) * H;
          }
          const rsrc_t ro = make_rsrc(dst, 32 * ld * 4);
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int n = tn0 + wn * WTN + j * 32 + lcol;  // column of the gradient
            const int nd = to_part ? n - tn0 : n;          // column in the destination
            u32x4 old[4];
            if constexpr (decltype(accum)::value) {
#pragma unroll
              for (int b = 0; b < 4; ++b)
                old[b] = load_b128(ro, n < ncols ? 4u * static_cast<uint32_t>((8 * b + hrow) * ld + nd) : kNoWrite);
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              float v[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * b + q];
              quad_transpose(v, lane);
              if constexpr (decltype(accum)::value) {
                v[0] += __uint_as_float(old[b].x);
                v[1] += __uint_as_float(old[b].y);
                v[2] += __uint_as_float(old[b].z);
                v[3] += __uint_as_float(old[b].w);
              }
              const uint32_t off = n < ncols ? 4u * static_cast<uint32_t>((8 * b + hrow) * ld + nd) : kNoWrite;
              store_b128(u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])},
                         ro, off);
            }
          }
        }
      };
      if (!to_part && P.accumulate != 0) store_blocks(std::true_type{});
      else store_blocks(std::false_type{});
    }
  };

  // ---- tile loop ---------------------------------------------------------------
  // Steps of a tile come in groups of NSTAGE (a padded step reads zeros), so
  // step u of a group always uses stage u and every stage is a distinct
  // object at compile time. In step s the loads of step s + 3 go out; in a
  // tile's last group they turn into the next tile's steps 0-2.
  int L = lo + slot;
  if (L < hi) {
    set_tile_and_offsets(L);
    if constexpr (GATHER_K) {
      // The tokens of step 4 go out between steps 1 and 2, as in the steady
      // state (one token load between two steps' operand loads): the first
      // k-step's wait for step 1 counts 14 newer loads (GATHER_K: kWaitVm14),
      // and with all five token loads ahead of step 0 only 13 would follow
      // step 1, so step 1's last block could still be in flight when its
      // fragments are read.
      // The scheduling barriers keep the compiler from moving the token
      // loads, whose place the count relies on.
      const uint32_t tk0 = load_tok(0), tk1 = load_tok(1), tk2 = load_tok(2);
      tkA = load_tok(3);
      __builtin_amdgcn_sched_barrier(0);
      gather_off(tk0, 0);
      issue(0, lds0);
      gather_off(tk1, 1);
      issue(1, lds1);
      __builtin_amdgcn_sched_barrier(0);
      tkB = load_tok(4);
      __builtin_amdgcn_sched_barrier(0);
      gather_off(tk2, 2);
      issue(2, lds2);
    } else {
      issue(0, lds0);
      issue(1, lds1);
      issue(2, lds2);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm16);  // step 0 has landed (steps 1 and 2 may not have)
    step_barrier();
  }
  for (; L < hi; L += nslots) {
    if constexpr (F8) {
      set_frag_offsets8();
      load_scales8();
      read_first8(std::integral_constant<int, FM>{}, lds0);
    } else {
      set_frag_offsets();
      read_slice(std::integral_constant<int, FM>{}, lds0, 0, fa0, fb0);
    }
    // This wavefront's 32-row blocks that hold valid rows of the tile (a
    // ragged last tile of an expert skips the MFMAs, fragment reads and
    // stores of the others). The k-loop is compiled once per count, so no
    // branch sits between the MFMAs.
    const int mrows_valid = grouped_k(MODE) ? (MODE == WGRAD_DOWN ? H : 2 * I) - m0 : mvalid;
    const int nbm = __builtin_amdgcn_readfirstlane(max(0, min(FM, (mrows_valid - wm * WTM + 31) / 32)));
    const int nsteps = max(NSTAGE, (ksteps + NSTAGE - 1) / NSTAGE * NSTAGE);
    const int fe = e, frow0 = row0, fmvalid = mvalid, fm0 = m0, fn0 = n0, fp = pidx;
    const int Lnext = L + nslots;
    constexpr std::false_type no{};
    constexpr bool EPI_PER_VARIANT = MODE == GATEUP && !F8;
    auto kst = [&](auto nbc, auto first, const bf16_t* Ac, const bf16_t* An, int sn, bf16_t* Ln, bool last)
                   __attribute__((always_inline)) {
      if constexpr (F8) kstep8(nbc, first, Ac, An, sn, Ln, last);
      else kstep(nbc, first, Ac, An, sn, Ln, last);
    };
    auto kloop = [&](auto nbc) __attribute__((always_inline)) {
      kst(nbc, std::true_type{}, lds0, lds1, 3, lds3, false);  // step 0: accumulators start at zero
      for (int s = NSTAGE; s < nsteps; s += NSTAGE) {         // steps s - 3 .. s
        kst(nbc, no, lds1, lds2, s, lds0, false);
        kst(nbc, no, lds2, lds3, s + 1, lds1, false);
        kst(nbc, no, lds3, lds0, s + 2, lds2, false);
        kst(nbc, no, lds0, lds1, s + 3, lds3, false);
      }
      if (Lnext < hi) set_tile_and_offsets(Lnext);
      else clear_tile();
      kst(nbc, no, lds1, lds2, 0, lds0, false);
      kst(nbc, no, lds2, lds3, 1, lds1, false);
      kst(nbc, no, lds3, lds0, 2, lds2, true);
      // The bf16 gate/up epilogue inside each variant: blocks without valid
      // rows are dead there, which leaves it without register spills (shared
      // behind the switch it spills; the other modes do best shared).
      if constexpr (EPI_PER_VARIANT) epilogue(fe, frow0, fmvalid, fm0, fn0, decltype(nbc)::value, fp);
    };
    switch (nbm) {
      case 4: kloop(std::integral_constant<int, 4>{}); break;
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      case 1: kloop(std::integral_constant<int, 1>{}); break;
      default: kloop(std::integral_constant<int, 0>{}); break;
    }
    if constexpr (!EPI_PER_VARIANT) epilogue(fe, frow0, fmvalid, fm0, fn0, nbm, fp);
    // The next tile's first steps have landed (everything this wavefront
    // issued has: loads and the epilogue's stores, which the counter does
    // not order against each other) in every wavefront, and all are done
    // with the last stages.
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    step_barrier();
    // The offsets again rather than kept alive through the epilogue (the
    // opaque lane index in set_offsets makes this a real recomputation).
    set_offsets(std::false_type{});
  }
}

template <int MODE, bool FUSED, bool F8, bool AW, bool F4, bool KX>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1))) void grouped_gemm_kernel(
    Params P) {
  MOE_GEMM_SMEM
  gemm_tiles<MODE, FUSED, F8, AW, F4, KX>(P, blockIdx.x, gridDim.x, sm);
}

// Two independent GEMMs of the backward in one persistent launch: a data
// gradient (A) and the weight gradient that reads the same inputs (B). Every
// workgroup runs its share of A, then its share of B: a workgroup that is
// done with A starts on B at once instead of waiting for A's slowest one,
// so only the launch's end has a tail. (Half the workgroups starting on B
// was measured too and was slower: each XCD then works on tiles twice as
// far apart, whose operands share its L2 less.)
template <int MA, int MB, bool FA, bool FB>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1))) void
grouped_gemm_pair_kernel(Params PA, Params PB) {
  MOE_GEMM_SMEM
  gemm_tiles<MA, FA>(PA, blockIdx.x, gridDim.x, sm);
  __syncthreads();  // the tables and stages are B's now
  gemm_tiles<MB, FB>(PB, blockIdx.x, gridDim.x, sm);
}

// Adds the partial tiles of every split expert into its weight gradient, in
// chunk order (chunk 0 is already there). Block b takes the split tiles b,
// b + grid, ...; the split plan is recomputed from the offsets exactly as the
// GEMM made it (same formulas, same GEMM grid).
template <int MODE>
__global__ __launch_bounds__(NT) void wgrad_reduce_kernel(Params P, int gemm_grid) {
  __shared__ int rstart[1025];  // first split tile of each expert (only split experts have any)
  __shared__ int pstart[1025];  // first partial tile of each expert
  __shared__ int part[NT];
  const int tid = threadIdx.x;
  const int H = P.H, E = P.E, I = P.I;
  const int mrows = MODE == WGRAD_DOWN ? H : 2 * I;
  const int ncols = MODE == WGRAD_DOWN ? I : H;
  const int ntn = (ncols + BN - 1) / BN;
  const int tpe = ((mrows + BM - 1) / BM) * ntn;
  int st[4], c[4], v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * 4 + j;
    st[j] = e < E ? (P.offsets[e + 1] - P.offsets[e] + BK - 1) / BK : 0;
  }
  expert_scan(st, rstart, part, E, tid);
  const int cap = split_cap(tpe * rstart[E], gemm_grid);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = tid * 4 + j < E ? split_chunks(st[j], cap) : 0;
    v[j] = c[j] > 1 ? tpe : 0;
  }
  expert_scan(v, rstart, part, E, tid);
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = c[j] > 0 ? (c[j] - 1) * tpe : 0;
  expert_scan(v, pstart, part, E, tid);
  const int R = rstart[E];
  for (int rt = blockIdx.x; rt < R; rt += gridDim.x) {
    int l2 = 0, h2 = E - 1;  // the split expert whose tiles hold rt
    while (l2 < h2) {
      const int mid = (l2 + h2 + 1) >> 1;
      if (rstart[mid] <= rt) l2 = mid; else h2 = mid - 1;
    }
    const int e = l2;
    const int t = rt - rstart[e];
    const int mt = t / ntn, nt = t - (t / ntn) * ntn;
    const int steps = (P.offsets[e + 1] - P.offsets[e] + BK - 1) / BK;
    const int chunks = split_chunks(steps, cap);
    for (int q = tid; q < BM * BN / 4; q += NT) {
      const int row = q / (BN / 4), c4 = (q - row * (BN / 4)) * 4;
      const int m = mt * BM + row, n = nt * BN + c4;
      if (m >= mrows || n >= ncols) continue;
      float* dst;
      if constexpr (MODE == WGRAD_DOWN) {
        dst = P.dw0 + (static_cast<int64_t>(e) * H + m) * I + n;
      } else {
        dst = m < I ? P.dw0 + (static_cast<int64_t>(e) * I + m) * H + n
                    : P.dw1 + (static_cast<int64_t>(e) * I + (m - I)) * H + n;
      }
      float4 sum = *reinterpret_cast<const float4*>(dst);
      for (int ch = 1; ch < chunks; ++ch) {
        const float4 pv = *reinterpret_cast<const float4*>(
            P.part + static_cast<int64_t>(pstart[e] + (ch - 1) * tpe + t) * (BM * BN) + row * BN + c4);
        sum.x += pv.x;
        sum.y += pv.y;
        sum.z += pv.z;
        sum.w += pv.w;
      }
      *reinterpret_cast<float4*>(dst) = sum;
    }
  }
}

template <int MODE>
hipError_t launch_wgrad_reduce(const Params& p, int grid, hipStream_t st) {
  // At most 2 * grid split tiles, two per reduction block at most.
  wgrad_reduce_kernel<MODE><<<grid, NT, 0, st>>>(p, grid);
  return hipGetLastError();
}

int persistent_grid() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
      cus = 256;
    cached = (cus / 8) * 8;
  }
  return cached;
}

template <int MODE, bool FUSED = false, bool F8 = false, bool AW = false, bool F4 = false, bool KX = false>
hipError_t run(const Params& p, hipStream_t st) {
  const int grid = persistent_grid();
  grouped_gemm_kernel<MODE, FUSED, F8, AW, F4, KX><<<grid, NT, 0, st>>>(p);
  hipError_t err = hipGetLastError();
  if constexpr (grouped_k(MODE)) {
    if (err != hipSuccess) return err;
    err = launch_wgrad_reduce<MODE>(p, grid, st);
  }
  return err;
}

template <int MA, int MB, bool FA = false, bool FB = false>
hipError_t run_pair(const Params& pa, const Params& pb, hipStream_t st) {
  const int grid = persistent_grid();
  grouped_gemm_pair_kernel<MA, MB, FA, FB><<<grid, NT, 0, st>>>(pa, pb);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_wgrad_reduce<MB>(pb, grid, st);
}

Params make_params(const moe_shape& s, const GemmArgs& g) {
  Params p{};
  p.T = s.T;
  p.M = s.T * s.k;
  p.H = s.H;
  p.E = s.E;
  p.I = s.I;
  p.offsets = g.offsets;
  p.a = static_cast<const bf16_t*>(g.a);
  p.b0 = static_cast<const bf16_t*>(g.b0);
  p.b1 = static_cast<const bf16_t*>(g.b1);
  p.g_in = static_cast<const bf16_t*>(g.g_in);
  p.u_in = static_cast<const bf16_t*>(g.u_in);
  p.out0 = static_cast<bf16_t*>(g.out0);
  p.out1 = static_cast<bf16_t*>(g.out1);
  p.out2 = static_cast<bf16_t*>(g.out2);
  p.out3 = static_cast<bf16_t*>(g.out3);
  p.dw0 = g.dw0;
  p.dw1 = g.dw1;
  p.accumulate = g.accumulate;
  p.part = g.part;
  p.row_token = g.row_token;
  p.row_weight = g.row_weight;
  p.sa = g.a_scale;
  p.sb0 = g.b0_scale;
  p.sb1 = g.b1_scale;
  p.ax = static_cast<const bf16_t*>(g.ax);
  p.bx0 = static_cast<const bf16_t*>(g.bx0);
  p.bx1 = static_cast<const bf16_t*>(g.bx1);
  p.kx = g.kx;
  p.kxr = g.kxr;
  p.kxp = g.kxp;
  return p;
}

}  // namespace

int gemm_grid() { return persistent_grid(); }

int64_t wgrad_part_tiles(const moe_shape& s) {
  if (s.dtype != MOE_BF16) return 0;
  const int64_t tpe_max = static_cast<int64_t>(ceil_div(2 * s.I, BM)) * ceil_div(s.H, BN);
  const int64_t steps = static_cast<int64_t>(s.T) * s.k / BK + s.E;  // >= the sum over experts of ceil(n_e / BK)
  return std::min<int64_t>(2 * static_cast<int64_t>(persistent_grid()), tpe_max * (steps / kMinChunkSteps));
}

hipError_t launch_gemm_bf16(GemmMode mode, const moe_shape& s, const GemmArgs& g, hipStream_t st) {
  const Params p = make_params(s, g);
  switch (mode) {
    case GEMM_GATEUP:
      if (g.kx > 0) {
        if (g.a_scale || g.out3) return hipErrorInvalidValue;
        return g.row_token ? run<GATEUP, true, false, false, false, true>(p, st)
                           : run<GATEUP, false, false, false, false, true>(p, st);
      }
      if (g.a_scale && g.b_fp4) return g.row_token ? run<GATEUP, true, true, false, true>(p, st) : hipErrorInvalidValue;
      if (g.a_scale) return g.row_token ? run<GATEUP, true, true>(p, st) : hipErrorInvalidValue;
      if (g.out3)  // a_w (needs row_weight)
        return g.row_token ? run<GATEUP, true, false, true>(p, st) : run<GATEUP, false, false, true>(p, st);
      return g.row_token ? run<GATEUP, true>(p, st) : run<GATEUP>(p, st);
    case GEMM_DOWN:
      if (g.kx > 0)
        return g.row_weight || g.a_scale ? hipErrorInvalidValue : run<DOWN, false, false, false, false, true>(p, st);
      if (g.a_scale && g.b_fp4) return g.row_weight ? run<DOWN, true, true, false, true>(p, st) : hipErrorInvalidValue;
      if (g.a_scale) return g.row_weight ? run<DOWN, true, true>(p, st) : hipErrorInvalidValue;
      return g.row_weight ? run<DOWN, true>(p, st) : run<DOWN>(p, st);
    case GEMM_DGRAD_DOWN:
      if (g.kx > 0)
        return g.row_token ? run<DGRAD_DOWN, true, false, false, false, true>(p, st)
                           : run<DGRAD_DOWN, false, false, false, false, true>(p, st);
      return g.row_token ? run<DGRAD_DOWN, true>(p, st) : run<DGRAD_DOWN>(p, st);
    case GEMM_DGRAD_GATEUP:
      if (g.kx > 0) return run<DGRAD_GATEUP, false, false, false, false, true>(p, st);
      return run<DGRAD_GATEUP>(p, st);
    case GEMM_WGRAD_DOWN: return g.row_token ? run<WGRAD_DOWN, true>(p, st) : run<WGRAD_DOWN>(p, st);
    case GEMM_WGRAD_GATEUP: return g.row_token ? run<WGRAD_GATEUP, true>(p, st) : run<WGRAD_GATEUP>(p, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_pair_bf16(GemmMode ma, GemmMode mb, const moe_shape& s, const GemmArgs& ga, const GemmArgs& gb,
                                 hipStream_t st) {
  const Params pa = make_params(s, ga), pb = make_params(s, gb);
  if (ma == GEMM_DGRAD_DOWN && mb == GEMM_WGRAD_DOWN) {
    if ((ga.row_token == nullptr) != (gb.row_token == nullptr)) return hipErrorInvalidValue;
    return ga.row_token ? run_pair<DGRAD_DOWN, WGRAD_DOWN, true, true>(pa, pb, st)
                        : run_pair<DGRAD_DOWN, WGRAD_DOWN>(pa, pb, st);
  }
  if (ma == GEMM_DGRAD_GATEUP && mb == GEMM_WGRAD_GATEUP)
    return gb.row_token ? run_pair<DGRAD_GATEUP, WGRAD_GATEUP, false, true>(pa, pb, st)
                        : run_pair<DGRAD_GATEUP, WGRAD_GATEUP>(pa, pb, st);
  return hipErrorInvalidValue;
}

}  // namespace moe
