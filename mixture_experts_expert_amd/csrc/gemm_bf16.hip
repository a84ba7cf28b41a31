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
// file (256 fp32 per lane). Operands go global -> registers -> LDS (two
// stages, 128 KiB) with the next k-step's global loads in flight while the
// current one multiplies. Both operands sit in LDS as [row][k] with k
// contiguous, in 16-byte chunks XOR-swizzled by row so the MFMA operand
// reads (32 rows at one k-chunk) hit distinct banks. Operands whose k is the
// strided index (data-gradient weights, both weight-gradient operands) are
// transposed in registers on their way into LDS (4 k-rows x 8 columns per
// thread).
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

// Physical element offset of 16-byte chunk `c` of LDS row `r`.
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ ((r ^ (r >> 3)) & 7)) << 3); }

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// Operand with k contiguous in memory: R rows x BK, one 16-byte chunk per
// (row, chunk) pair; thread t owns chunks t + i*NT, i.e. row i*(NT/CH) + t/CH,
// chunk t % CH.
template <int R>
struct KLoader {
  static constexpr int N = R * CH / NT;
  const bf16_t* base[N];
  int off[N];
  u32x4 v[N];
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = *reinterpret_cast<const u32x4*>(base[i] + off[i] + k0);
  }
  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
    const int c = tid % CH;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = i * (NT / CH) + tid / CH;
      *reinterpret_cast<u32x4*>(lds + swz(r, c)) = v[i];
    }
  }
};

// Operand with k strided in memory ([k][mn], mn contiguous): blocks of 4
// k-rows x 8 columns; thread t owns blocks q = t + i*NT with kb = q % 16
// (k-rows 4kb..4kb+3 of the step) and mb = q / 16 (columns 8mb..8mb+7).
// Rows at or past `rows_left` read as zero (ragged reductions).
template <int R>
struct TLoader {
  static constexpr int N = 2 * R / NT;
  int off[N];  // (4*kb)*ld + first column of the block
  u32x4 v[N][4];
  __device__ __forceinline__ void load(const bf16_t* base, int ld, int rows_left, int tid) {
    const int kb = tid % 16;
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int kr = 0; kr < 4; ++kr) {
        const int row = kb * 4 + kr;
        u32x4 z = {0u, 0u, 0u, 0u};
        if (row < rows_left) z = *reinterpret_cast<const u32x4*>(base + off[i] + kr * ld);
        v[i][kr] = z;
      }
  }
  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
    const int kb = tid % 16;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int mb = (tid + i * NT) / 16;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int w = c >> 1;
        u32x2 o;
        if (c & 1) {
          o.x = hi_pair(v[i][0][w], v[i][1][w]);
          o.y = hi_pair(v[i][2][w], v[i][3][w]);
        } else {
          o.x = lo_pair(v[i][0][w], v[i][1][w]);
          o.y = lo_pair(v[i][2][w], v[i][3][w]);
        }
        const int r = mb * 8 + c;
        *reinterpret_cast<u32x2*>(lds + swz(r, kb >> 1) + ((kb & 1) << 2)) = o;
      }
    }
  }
};

__device__ __forceinline__ float bf(bf16_t v) { return bf16_to_f32(v); }

template <int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1))) void grouped_gemm_kernel(
    Params P) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * STAGE];
  __shared__ int tstart[1025];  // grouped-M: first m-tile of each expert
  __shared__ int part[NT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  KLoader<BM> ka;   // A, k contiguous (grouped-M)
  TLoader<BM> ta;   // A, k strided (grouped-K)
  KLoader<BN> kb;   // B, k contiguous (GATEUP, DOWN)
  TLoader<BN> tb;   // B, k strided (data and weight gradients)

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

    // ---- per-tile operand addressing ----------------------------------------
    int ksteps;
    int lda = 0, ldb = 0;
    if constexpr (MODE == GATEUP) { lda = H; ksteps = H / BK; }
    if constexpr (MODE == DOWN) { lda = I; ksteps = I / BK; }
    if constexpr (MODE == DGRAD_DOWN) { lda = H; ldb = I; ksteps = H / BK; }
    if constexpr (MODE == DGRAD_GATEUP) { lda = 2 * I; ldb = H; ksteps = 2 * I / BK; }
    if constexpr (MODE == WGRAD_DOWN) { lda = H; ldb = I; ksteps = (kend - kbeg + BK - 1) / BK; }
    if constexpr (MODE == WGRAD_GATEUP) { lda = 2 * I; ldb = H; ksteps = (kend - kbeg + BK - 1) / BK; }

    if constexpr (!grouped_k(MODE)) {
      const bf16_t* abase = P.a + static_cast<int64_t>(row0) * lda;
#pragma unroll
      for (int i = 0; i < KLoader<BM>::N; ++i) {
        const int r = i * (NT / CH) + tid / CH;
        ka.off[i] = min(r, mvalid - 1) * lda + (tid % CH) * 8;
        ka.base[i] = abase;
      }
    } else {
      const int mrows = MODE == WGRAD_DOWN ? H : 2 * I;
#pragma unroll
      for (int i = 0; i < TLoader<BM>::N; ++i) {
        const int q = tid + i * NT;
        const int col = min(m0 + (q / 16) * 8, mrows - 8);
        ta.off[i] = (q % 16) * 4 * lda + col;
      }
    }
    if constexpr (MODE == GATEUP) {
      const int64_t ebase = static_cast<int64_t>(e) * I * H;
#pragma unroll
      for (int i = 0; i < KLoader<BN>::N; ++i) {
        // LDS row r = 32 i + tid / 8; wavefront column half wn = i / 4 and
        // 32-column block j = i % 4 (j < 2: gate, j >= 2: up) of that half.
        const int j = i % 4, half = i / 4;
        const int idx = min(n0 + half * 64 + (j & 1) * 32 + tid / CH, I - 1);
        kb.off[i] = idx * H + (tid % CH) * 8;
        kb.base[i] = (j < 2 ? P.b0 : P.b1) + ebase;
      }
    }
    if constexpr (MODE == DOWN) {
      const bf16_t* bbase = P.b0 + static_cast<int64_t>(e) * H * I;
#pragma unroll
      for (int i = 0; i < KLoader<BN>::N; ++i) {
        const int r = i * (NT / CH) + tid / CH;
        kb.off[i] = min(n0 + r, H - 1) * I + (tid % CH) * 8;
        kb.base[i] = bbase;
      }
    }
    if constexpr (!b_kcontig(MODE)) {
      const int ncols = (MODE == DGRAD_DOWN || MODE == WGRAD_DOWN) ? I : H;
#pragma unroll
      for (int i = 0; i < TLoader<BN>::N; ++i) {
        const int q = tid + i * NT;
        const int col = min(n0 + (q / 16) * 8, ncols - 8);
        tb.off[i] = (q % 16) * 4 * ldb + col;
      }
    }

    // k-step s: global loads of A and B into registers.
    auto load_step = [&](int s) {
      const int k0 = s * BK;
      if constexpr (!grouped_k(MODE)) {
        ka.load(k0);
      } else {
        ta.load(P.a + static_cast<int64_t>(kbeg + k0) * lda, lda, kend - kbeg - k0, tid);
      }
      if constexpr (b_kcontig(MODE)) {
        kb.load(k0);
      } else if constexpr (MODE == DGRAD_DOWN) {
        tb.load(P.b0 + static_cast<int64_t>(e) * H * I + static_cast<int64_t>(k0) * I, ldb, BK, tid);
      } else if constexpr (MODE == DGRAD_GATEUP) {
        const bf16_t* base = k0 < I ? P.b0 + static_cast<int64_t>(e) * I * H + static_cast<int64_t>(k0) * H
                                    : P.b1 + static_cast<int64_t>(e) * I * H + static_cast<int64_t>(k0 - I) * H;
        tb.load(base, ldb, BK, tid);
      } else {
        tb.load(P.b0 + static_cast<int64_t>(kbeg + k0) * ldb, ldb, kend - kbeg - k0, tid);
      }
    };
    auto store_step = [&](int stage) {
      bf16_t* As = lds + stage * STAGE;
      bf16_t* Bs = As + STAGE_A;
      if constexpr (!grouped_k(MODE)) ka.store(As, tid); else ta.store(As, tid);
      if constexpr (b_kcontig(MODE)) kb.store(Bs, tid); else tb.store(Bs, tid);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    if (ksteps > 0) {
      load_step(0);
      store_step(0);
      __syncthreads();
      for (int s = 0; s < ksteps; ++s) {
        if (s + 1 < ksteps) load_step(s + 1);
        const bf16_t* As = lds + (s & 1) * STAGE;
        const bf16_t* Bs = As + STAGE_A;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
          const int c = kk * 2 + (lane >> 5);
          bf16x8 av[FM], bv[FN];
#pragma unroll
          for (int i = 0; i < FM; ++i)
            av[i] = *reinterpret_cast<const bf16x8*>(As + swz(wm * WTM + i * 32 + (lane & 31), c));
#pragma unroll
          for (int j = 0; j < FN; ++j)
            bv[j] = *reinterpret_cast<const bf16x8*>(Bs + swz(wn * WTN + j * 32 + (lane & 31), c));
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        if (s + 1 < ksteps) store_step((s + 1) & 1);
        __syncthreads();
      }
    }

    // ---- epilogue -------------------------------------------------------------
    // acc[i][j][q] holds tile row wm*128 + i*32 + 8*(q/4) + 4*(lane/32) + q%4,
    // tile column wn*128 + j*32 + lane%32.
    const int rbase = wm * WTM + 4 * (lane >> 5);
    const int cl = lane & 31;
    if constexpr (MODE == GATEUP) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int idx = n0 + wn * 64 + jj * 32 + cl;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int tr = rbase + i * 32 + 8 * (q >> 2) + (q & 3);
            if (tr < mvalid && idx < I) {
              const int64_t o = static_cast<int64_t>(row0 + tr) * I + idx;
              const float gv = acc[i][jj][q], uv = acc[i][jj + 2][q];
              P.out0[o] = f32_to_bf16(gv);
              P.out1[o] = f32_to_bf16(uv);
              P.out2[o] = f32_to_bf16(gv * sigmoidf_dev(gv) * uv);
            }
          }
        }
    } else if constexpr (MODE == DOWN || MODE == DGRAD_GATEUP) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int n = n0 + wn * WTN + j * 32 + cl;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int tr = rbase + i * 32 + 8 * (q >> 2) + (q & 3);
            if (tr < mvalid && n < H) P.out0[static_cast<int64_t>(row0 + tr) * H + n] = f32_to_bf16(acc[i][j][q]);
          }
        }
    } else if constexpr (MODE == DGRAD_DOWN) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int idx = n0 + wn * WTN + j * 32 + cl;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int tr = rbase + i * 32 + 8 * (q >> 2) + (q & 3);
            if (tr < mvalid && idx < I) {
              const int64_t p = row0 + tr;
              const float gv = bf(P.g_in[p * I + idx]), uv = bf(P.u_in[p * I + idx]);
              const float sg = sigmoidf_dev(gv);
              const float da = acc[i][j][q];
              P.out0[p * 2 * I + idx] = f32_to_bf16(da * uv * sg * (1.0f + gv * (1.0f - sg)));
              P.out0[p * 2 * I + I + idx] = f32_to_bf16(da * (gv * sg));
            }
          }
        }
    } else {
      const int mrows = MODE == WGRAD_DOWN ? H : 2 * I;
      const int ncols = MODE == WGRAD_DOWN ? I : H;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int n = n0 + wn * WTN + j * 32 + cl;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int m = m0 + rbase + i * 32 + 8 * (q >> 2) + (q & 3);
            if (m < mrows && n < ncols) {
              float* dst;
              if constexpr (MODE == WGRAD_DOWN) {
                dst = P.dw0 + (static_cast<int64_t>(e) * H + m) * I + n;
              } else {
                dst = m < I ? P.dw0 + (static_cast<int64_t>(e) * I + m) * H + n
                            : P.dw1 + (static_cast<int64_t>(e) * I + (m - I)) * H + n;
              }
              *dst = P.accumulate ? *dst + acc[i][j][q] : acc[i][j][q];
            }
          }
        }
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
