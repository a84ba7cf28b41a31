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
// Tile: 256 x 256 x 64 per workgroup of 4 wavefronts (2 x 2), 128 x 128 per
// wavefront as 4 x 4 MFMA blocks of 32 x 32, accumulators in the register
// file (256 fp32 per lane). Operands go straight from global memory into LDS
// (global_load_lds_dwordx4: each wavefront instruction fills one contiguous
// KiB, lane l at byte 16 l), two stages of 64 KiB, the next k-step's loads in
// flight while the current one multiplies; no register staging and no LDS
// store phase. An operand whose reduction index is contiguous in memory
// ("k-major": the forward operands, the data-gradient activations) sits in
// LDS as [row][k], 16-byte chunks XOR-swizzled by row, and is read with
// ds_read_b128. An operand whose reduction index is the strided one
// ("mn-major": the data-gradient weights, both weight-gradient operands) sits
// as [k][column] as it is in memory, chunks swizzled by k, and is read with
// ds_read_b64_tr_b16, which hands each lane four consecutive k of one column
// (within each 16-lane group, lane i receives element i%4 of the pieces that
// lanes 4j + i/4 address). Either way the swizzle is applied on the global
// side: each lane fetches the chunk that belongs at its fixed LDS slot.
//
// Scheduling: one workgroup per CU, persistent. Tile i of the list belongs
// to XCD-local workgroups: the list is cut into 8 contiguous ranges, one per
// XCD (workgroup b runs on XCD b % 8), and the tiles of one expert and one
// column block sit next to each other, so the weight slice they share is
// fetched into one XCD's L2 once.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NT = 256;                 // threads per workgroup
constexpr int WTM = 128, WTN = 128;     // wavefront tile
constexpr int FM = WTM / 32, FN = WTN / 32;
constexpr int CH = BK / 8;              // 16-byte chunks per LDS row
constexpr int STAGE_A = BM * BK;        // bf16 elements
constexpr int STAGE_B = BN * BK;
constexpr int STAGE = STAGE_A + STAGE_B;
constexpr int GU_COLS = BN / 2;         // intermediate columns per GATEUP tile (gate + up)

enum Mode : int { GATEUP = 0, DOWN = 1, DGRAD_DOWN = 2, DGRAD_GATEUP = 3, WGRAD_DOWN = 4, WGRAD_GATEUP = 5 };

constexpr bool grouped_k(int m) { return m >= WGRAD_DOWN; }
constexpr bool b_kcontig(int m) { return m == GATEUP || m == DOWN; }

struct Params {
  int H, E, I;
  const int32_t* offsets;
  const bf16_t* a;     // x_perm | act | do_perm | dgu | do_perm | dgu
  const bf16_t* b0;    // w_gate | w_down | w_down | w_gate | act | x_perm
  const bf16_t* b1;    // w_up (GATEUP, DGRAD_GATEUP)
  const bf16_t* g_in;  // DGRAD_DOWN: saved g
  const bf16_t* u_in;  // DGRAD_DOWN: saved u
  bf16_t* out0;        // g | o_perm | dgu | dx_perm
  bf16_t* out1;        // u (GATEUP)
  bf16_t* out2;        // a (GATEUP)
  float* dw0;          // dw_down | dw_gate
  float* dw1;          // dw_up
  int accumulate;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// LDS layouts of one operand stage (bf16 elements):
//   k-major  [256 rows][64 k]   chunk c of row r at r*64 + (c ^ swk(r))*8
//   mn-major [64 k][256 cols]   chunk c of row k at k*256 + (c ^ swt(k))*8
__device__ __forceinline__ int swk(int r) { return (r ^ (r >> 3)) & 7; }
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
// L2 prefetch: one dword per lane (one per 128-byte line) dropped into a
// scratch LDS slot that nothing reads; it has no register destination, so it
// can stay in flight across k-steps.
__device__ __forceinline__ void buf_prefetch(rsrc_t r, uint32_t voff, uint32_t* sink) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)sink, 4, voff, 0, 0, 0);
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
// [6:4], lgkmcnt in [11:8]. Both wait for LDS traffic and for all but the
// newest `n` vector-memory instructions (expcnt left unconstrained).
constexpr int kWaitVm0 = 0x0070;  // vmcnt(0) lgkmcnt(0)
constexpr int kWaitVm2 = 0x0072;  // vmcnt(2) lgkmcnt(0)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Four floats -> four bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  const f32x2 lo = {a, b}, hi = {c, d};
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                    __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2)));
}

template <int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1))) void grouped_gemm_kernel(
    Params P) {
  // Two stages as two objects: with the stage of every access known at
  // compile time, the compiler sees that loads landing in one stage do not
  // alias reads of the other and does not wait for them before reading.
  __shared__ __attribute__((aligned(16))) bf16_t lds0[STAGE];
  __shared__ __attribute__((aligned(16))) bf16_t lds1[STAGE];
  __shared__ int tstart[1025];  // grouped-M: first m-tile of each expert
  __shared__ uint32_t pf_sink[4 * 64];  // L2-prefetch landing slots, never read
  __shared__ int part[NT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  const int wm = wave >> 1, wn = wave & 1;
  const int H = P.H, E = P.E, I = P.I;

  // ---- tile list -----------------------------------------------------------
  int ntn, total;
  int tpe = 0;
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
    const int mrows = MODE == WGRAD_DOWN ? H : 2 * I;
    const int ncols = MODE == WGRAD_DOWN ? I : H;
    ntn = (ncols + BN - 1) / BN;
    tpe = ((mrows + BM - 1) / BM) * ntn;
    total = E * tpe;
  }

  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int nslots = gridDim.x >> 3;
  const int lo = static_cast<int>((static_cast<int64_t>(total) * xcd) / 8);
  const int hi = static_cast<int>((static_cast<int64_t>(total) * (xcd + 1)) / 8);

  constexpr bool A_KMAJOR = !grouped_k(MODE);
  constexpr bool B_KMAJOR = b_kcontig(MODE);

  for (int L = lo + slot; L < hi; L += nslots) {
    // ---- decode the tile ---------------------------------------------------
    int e, row0 = 0, mvalid = 0, m0 = 0, n0 = 0, nt = 0, kbeg = 0, kend = 0;
    if constexpr (!grouped_k(MODE)) {
      int l2 = 0, h2 = E - 1;
      while (l2 < h2) {
        const int mid = (l2 + h2 + 1) >> 1;
        if (tstart[mid] * ntn <= L) l2 = mid; else h2 = mid - 1;
      }
      e = l2;
      const int rem = L - tstart[e] * ntn;
      const int mte = tstart[e + 1] - tstart[e];
      nt = rem / mte;
      const int mt = rem - nt * mte;
      row0 = P.offsets[e] + mt * BM;
      mvalid = min(BM, P.offsets[e + 1] - row0);
      n0 = nt * (MODE == GATEUP ? GU_COLS : BN);
    } else {
      e = L / tpe;
      const int rem = L - e * tpe;
      const int mt = rem / ntn;
      nt = rem - mt * ntn;
      m0 = mt * BM;
      n0 = nt * BN;
      kbeg = P.offsets[e];
      kend = P.offsets[e + 1];
    }

    // The decode is the same on every lane; say so, so that the operand
    // bases live in scalar registers and the loads use the scalar-base form.
    e = __builtin_amdgcn_readfirstlane(e);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    mvalid = __builtin_amdgcn_readfirstlane(mvalid);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    n0 = __builtin_amdgcn_readfirstlane(n0);
    kbeg = __builtin_amdgcn_readfirstlane(kbeg);
    kend = __builtin_amdgcn_readfirstlane(kend);

    int ksteps, lda = 0, ldb = 0;
    if constexpr (MODE == GATEUP) { lda = H; ksteps = H / BK; }
    if constexpr (MODE == DOWN) { lda = I; ksteps = I / BK; }
    if constexpr (MODE == DGRAD_DOWN) { lda = H; ldb = I; ksteps = H / BK; }
    if constexpr (MODE == DGRAD_GATEUP) { lda = 2 * I; ldb = H; ksteps = 2 * I / BK; }
    if constexpr (MODE == WGRAD_DOWN) { lda = H; ldb = I; ksteps = (kend - kbeg + BK - 1) / BK; }
    if constexpr (MODE == WGRAD_GATEUP) { lda = 2 * I; ldb = H; ksteps = (kend - kbeg + BK - 1) / BK; }

    // ---- per-lane byte offsets of this wavefront's 8 + 8 load instructions,
    // relative to the operand's base at the current k-step; instruction t
    // fills LDS block wave*8 + t (1 KiB) of each operand stage. Rows and
    // columns past the operand's end are clamped to its last one (their
    // products land in rows or columns that are never stored). k-major:
    // LDS row r = 8 (wave*8 + t) + lane/8, chunk lane%8 (swizzled). mn-major:
    // k-row 2 (wave*8 + t) + lane/32, chunk lane%32 (swizzled).
    uint32_t aoff[8], boff[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int blk = wave * 8 + t;
      if constexpr (A_KMAJOR) {
        const int r = blk * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swk(r);
        aoff[t] = 2u * (min(r, mvalid - 1) * lda + c * 8);
      } else {
        const int k = blk * 2 + (lane >> 5);
        const int c = (lane & 31) ^ swt(k);
        const int mrows = MODE == WGRAD_DOWN ? H : 2 * I;
        aoff[t] = 2u * (k * lda + min(m0 + c * 8, mrows - 8));
      }
      if constexpr (MODE == GATEUP) {
        // LDS row r: wavefront column half r / 128 and 32-column block
        // j = (r % 128) / 32 of it (j < 2: gate, j >= 2: up, same indices).
        // A wavefront's 64 rows are all gate (even waves) or all up (odd).
        const int r = blk * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swk(r);
        const int j = (r & 127) >> 5;
        const int idx = min(n0 + (r >> 7) * 64 + (j & 1) * 32 + (r & 31), I - 1);
        boff[t] = 2u * (idx * H + c * 8);
      } else if constexpr (MODE == DOWN) {
        const int r = blk * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swk(r);
        boff[t] = 2u * (min(n0 + r, H - 1) * I + c * 8);
      } else {
        const int k = blk * 2 + (lane >> 5);
        const int c = (lane & 31) ^ swt(k);
        const int ncols = (MODE == DGRAD_DOWN || MODE == WGRAD_DOWN) ? I : H;
        boff[t] = 2u * (k * ldb + min(n0 + c * 8, ncols - 8));
      }
    }
    const bf16_t* abase_m = P.a + static_cast<int64_t>(row0) * lda;  // grouped-M A

    // L2 prefetch offsets, one 128-byte line per lane per operand and k-step:
    // k-major operands, row wave*64 + lane (its 64 k of the step); mn-major
    // operands, k-row wave*16 + lane/4, line lane%4 of the 256 columns.
    uint32_t pfa, pfb;
    {
      const int r = wave * 64 + lane;
      const int kr = wave * 16 + (lane >> 2);
      if constexpr (A_KMAJOR) {
        pfa = 2u * (min(r, mvalid - 1) * lda);
      } else {
        const int mrows = MODE == WGRAD_DOWN ? H : 2 * I;
        pfa = 2u * (kr * lda + min(m0 + (lane & 3) * 64, mrows - 64));
      }
      if constexpr (MODE == GATEUP) {
        const int j = (r & 127) >> 5;
        pfb = 2u * (min(n0 + (r >> 7) * 64 + (j & 1) * 32 + (r & 31), I - 1) * H);
      } else if constexpr (MODE == DOWN) {
        pfb = 2u * (min(n0 + r, H - 1) * I);
      } else {
        const int ncols = (MODE == DGRAD_DOWN || MODE == WGRAD_DOWN) ? I : H;
        pfb = 2u * (kr * ldb + min(n0 + (lane & 3) * 64, ncols - 64));
      }
    }
    uint32_t* sink = pf_sink + wave * 64;

    // Buffer resources of k-step s (num_records 0 past the last step).
    auto rsrc_a = [&](int s) -> rsrc_t {
      const int k0 = s * BK;
      if constexpr (A_KMAJOR) {
        return make_rsrc(abase_m + k0, s < ksteps ? 2 * (mvalid * lda - k0) : 0);
      } else {
        const int left = kend - kbeg - k0;
        return make_rsrc(P.a + static_cast<int64_t>(kbeg + k0) * lda, left > 0 ? 2 * left * lda : 0);
      }
    };
    auto rsrc_b = [&](int s) -> rsrc_t {
      const int k0 = s * BK;
      const bool live = s < ksteps;
      if constexpr (MODE == GATEUP) {
        const bf16_t* w = ((wave & 1) ? P.b1 : P.b0) + static_cast<int64_t>(e) * I * H + k0;
        return make_rsrc(w, live ? 2 * (I * H - k0) : 0);
      } else if constexpr (MODE == DOWN) {
        return make_rsrc(P.b0 + static_cast<int64_t>(e) * H * I + k0, live ? 2 * (H * I - k0) : 0);
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
        return make_rsrc(P.b0 + static_cast<int64_t>(kbeg + k0) * ldb, left > 0 ? 2 * left * ldb : 0);
      }
    };

    // Issue every load of k-step s into the stage at As, then the L2 prefetch
    // of step s + 1 (always exactly two more vector-memory instructions).
    auto issue = [&](int s, bf16_t* As) {
      bf16_t* Bs = As + STAGE_A;
      const rsrc_t ra = rsrc_a(s);
      const rsrc_t rb = rsrc_b(s);
#pragma unroll
      for (int t = 0; t < 8; ++t) buf_to_lds16(ra, aoff[t], As + (wave * 8 + t) * 512);
#pragma unroll
      for (int t = 0; t < 8; ++t) buf_to_lds16(rb, boff[t], Bs + (wave * 8 + t) * 512);
      buf_prefetch(rsrc_a(s + 1), pfa, sink);
      buf_prefetch(rsrc_b(s + 1), pfb, sink);
    };

    // Operand fragments of k-slice kk (16 k) for 32-row block i, as byte
    // offsets inside a stage. k-major (ds_read_b128, lane: row i*32 + lane%32,
    // chunk 2 kk + lane/32): the chunk XOR makes slice kk the slice-0 offset
    // XOR 32 kk. mn-major (two ds_read_b64_tr_b16, lane: k-row
    // 8 (lane/32) + (lane%16)/4, columns 4 (lane%4) .. + 3 of the block's
    // 16-column half (lane/16)%2): slice kk adds 16 rows = 8 KiB, the second
    // read 4 rows = 2 KiB.
    const int hi32 = lane >> 5;
    const int g16 = lane >> 4, i16 = lane & 15;
    int aof[FM], bof[FN];
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
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    // One k-step on the stage at As: operand fragments of k-slice kk + 1
    // are read while the 16 MFMAs of slice kk run; scheduling fences keep the
    // slices apart so the reads' latency runs under the matrix work.
    // Each k-step ends waiting for all but this wavefront's two newest
    // vector-memory instructions: the L2 prefetches, which may stay in flight.
    auto compute = [&](const bf16_t* As) {
      const bf16_t* Bs = As + STAGE_A;
      // Opaque to the optimiser: keeps the per-slice addresses below from
      // being hoisted out of the k-loop (for both stages and all slices,
      // which would not fit in registers).

      bf16x8 av[2][FM], bv[2][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) av[0][i] = frag(As, aof[i], 0, A_KMAJOR);
#pragma unroll
      for (int j = 0; j < FN; ++j) bv[0][j] = frag(Bs, bof[j], 0, B_KMAJOR);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int cur = kk & 1;
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 1 < BK / 16) {
#pragma unroll
          for (int i = 0; i < FM; ++i) av[cur ^ 1][i] = frag(As, aof[i], kk + 1, A_KMAJOR);
#pragma unroll
          for (int j = 0; j < FN; ++j) bv[cur ^ 1][j] = frag(Bs, bof[j], kk + 1, B_KMAJOR);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[cur][i], bv[cur][j], acc[i][j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitVm2);  // this wavefront's loads of the next step have landed ...
      step_barrier();                        // ... everyone's have, and this stage is free again
    };

    if (ksteps > 0) {
      issue(0, lds0);
      __builtin_amdgcn_s_waitcnt(kWaitVm2);
      step_barrier();
      // Steps go in pairs (stage 0, stage 1); an odd count gets one more
      // step, which reads as zeros (its buffer range is empty).
      const int ksteps2 = (ksteps + 1) & ~1;
      for (int s = 0; s < ksteps2; s += 2) {
        issue(s + 1, lds1);
        compute(lds0);
        if (s + 2 < ksteps2) issue(s + 2, lds0);
        compute(lds1);
      }
    }

    // ---- epilogue -------------------------------------------------------------
    // acc[i][j][q] holds wavefront-tile row i*32 + 8*(q/4) + 4*(lane/32) + q%4,
    // column j*32 + lane%32. Each 32-row block goes through this wavefront's
    // 16 KiB slice of LDS (fp32, [32][128]) and leaves as row-contiguous
    // vectors: 4 columns per lane, 32 lanes per 128-column row.
    float* stage = reinterpret_cast<float*>(lds0) + wave * (32 * WTN);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q)
          stage[(8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)) * WTN + j * 32 + (lane & 31)] = acc[i][j][q];
      __syncthreads();
      const int trow0 = wm * WTM + i * 32;  // tile row of stage row 0
      if constexpr (MODE == GATEUP) {
        // Columns 0..63 of the wavefront tile are gate, 64..127 up, for the
        // same 64 intermediate indices.
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int r = it * 4 + (lane >> 4);
          const int c = (lane & 15) * 4;
          const int tr = trow0 + r;
          const int idx = n0 + wn * 64 + c;
          if (tr < mvalid && idx < I) {
            const float4 gv = *reinterpret_cast<const float4*>(stage + r * WTN + c);
            const float4 uv = *reinterpret_cast<const float4*>(stage + r * WTN + 64 + c);
            const float av[4] = {gv.x * sigmoidf_dev(gv.x) * uv.x, gv.y * sigmoidf_dev(gv.y) * uv.y,
                                 gv.z * sigmoidf_dev(gv.z) * uv.z, gv.w * sigmoidf_dev(gv.w) * uv.w};
            const int64_t o = static_cast<int64_t>(row0 + tr) * I + idx;
            *reinterpret_cast<uint2*>(P.out0 + o) = pack_bf16x4(gv.x, gv.y, gv.z, gv.w);
            *reinterpret_cast<uint2*>(P.out1 + o) = pack_bf16x4(uv.x, uv.y, uv.z, uv.w);
            *reinterpret_cast<uint2*>(P.out2 + o) = pack_bf16x4(av[0], av[1], av[2], av[3]);
          }
        }
      } else {
#pragma unroll
        for (int it = 0; it < 16; ++it) {
          const int r = it * 2 + (lane >> 5);
          const int c = (lane & 31) * 4;
          const int tr = trow0 + r;
          const float4 v = *reinterpret_cast<const float4*>(stage + r * WTN + c);
          const int n = n0 + wn * WTN + c;
          if constexpr (MODE == DOWN || MODE == DGRAD_GATEUP) {
            if (tr < mvalid && n < H)
              *reinterpret_cast<uint2*>(P.out0 + static_cast<int64_t>(row0 + tr) * H + n) =
                  pack_bf16x4(v.x, v.y, v.z, v.w);
          } else if constexpr (MODE == DGRAD_DOWN) {
            if (tr < mvalid && n < I) {
              const int64_t p = row0 + tr;
              const uint2 gb = *reinterpret_cast<const uint2*>(P.g_in + p * I + n);
              const uint2 ub = *reinterpret_cast<const uint2*>(P.u_in + p * I + n);
              const float gv[4] = {__uint_as_float(gb.x << 16), __uint_as_float(gb.x & 0xffff0000u),
                                   __uint_as_float(gb.y << 16), __uint_as_float(gb.y & 0xffff0000u)};
              const float uv[4] = {__uint_as_float(ub.x << 16), __uint_as_float(ub.x & 0xffff0000u),
                                   __uint_as_float(ub.y << 16), __uint_as_float(ub.y & 0xffff0000u)};
              const float da[4] = {v.x, v.y, v.z, v.w};
              float dg[4], du[4];
#pragma unroll
              for (int e2 = 0; e2 < 4; ++e2) {
                const float sg = sigmoidf_dev(gv[e2]);
                dg[e2] = da[e2] * uv[e2] * sg * (1.0f + gv[e2] * (1.0f - sg));
                du[e2] = da[e2] * (gv[e2] * sg);
              }
              *reinterpret_cast<uint2*>(P.out0 + p * 2 * I + n) = pack_bf16x4(dg[0], dg[1], dg[2], dg[3]);
              *reinterpret_cast<uint2*>(P.out0 + p * 2 * I + I + n) = pack_bf16x4(du[0], du[1], du[2], du[3]);
            }
          } else {
            const int mrows = MODE == WGRAD_DOWN ? H : 2 * I;
            const int ncols = MODE == WGRAD_DOWN ? I : H;
            const int m = m0 + tr;
            if (m < mrows && n < ncols) {
              float* dst;
              if constexpr (MODE == WGRAD_DOWN) {
                dst = P.dw0 + (static_cast<int64_t>(e) * H + m) * I + n;
              } else {
                dst = m < I ? P.dw0 + (static_cast<int64_t>(e) * I + m) * H + n
                            : P.dw1 + (static_cast<int64_t>(e) * I + (m - I)) * H + n;
              }
              float4 o = v;
              if (P.accumulate) {
                const float4 old = *reinterpret_cast<const float4*>(dst);
                o.x += old.x;
                o.y += old.y;
                o.z += old.z;
                o.w += old.w;
              }
              *reinterpret_cast<float4*>(dst) = o;
            }
          }
        }
      }
      __syncthreads();  // the slice is rewritten by the next block (or the next tile's loads)
    }
  }
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

template <int MODE>
hipError_t run(const Params& p, hipStream_t st) {
  grouped_gemm_kernel<MODE><<<persistent_grid(), NT, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(GemmMode mode, const moe_shape& s, const GemmArgs& g, hipStream_t st) {
  Params p{};
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
  p.dw0 = g.dw0;
  p.dw1 = g.dw1;
  p.accumulate = g.accumulate;
  switch (mode) {
    case GEMM_GATEUP: return run<GATEUP>(p, st);
    case GEMM_DOWN: return run<DOWN>(p, st);
    case GEMM_DGRAD_DOWN: return run<DGRAD_DOWN>(p, st);
    case GEMM_DGRAD_GATEUP: return run<DGRAD_GATEUP>(p, st);
    case GEMM_WGRAD_DOWN: return run<WGRAD_DOWN>(p, st);
    case GEMM_WGRAD_GATEUP: return run<WGRAD_GATEUP>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
