// Expert indexing and gather: counts, offsets, the stable permutation of the
// T*k (token, slot) pairs by expert, and the gather of x into that order.
//
// The stable counting sort (unsloth PR #3812, review suggestion: a stable
// argsort of the flattened expert ids plus a bincount) runs in three passes
// over fixed blocks of kPermBlock pairs, with no atomics on positions:
//   1. per-block expert histograms (LDS integer atomics; counts only),
//   2. one block scans each expert's column of block counts (block bases and
//      counts) and the counts themselves (offsets); with at most 128 blocks
//      every block of pass 3 does this for itself instead, so two launches,
//   3. each block ranks its pairs in flat order: inside a wavefront the pairs
//      with the same expert are found by one ballot per bit of the expert id,
//      and a pair's rank is the number of such lanes below it; wavefronts and
//      chunks are ordered through per-expert counters in LDS.
// The position of pair f is offsets[e] + (pairs of expert e in earlier
// blocks) + (rank inside its block): the definition of the stable order.
#include <mutex>

#include "moe_internal.h"

// Device memory of the allocation-free sort (moe_forward_fused_noalloc): the
// per-block histograms live in this array instead of a caller's workspace.
// Each device holds its own copy for the life of the process; host code
// reaches it only through the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) int32_t scratch[moe::kScratchBytes / sizeof(int32_t)];

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kSlabInts = 8192;  // block counts staged in LDS per scan step
// Up to this many indexing blocks (T*k <= 131072 pairs), the ranking blocks
// scan the block counts themselves; past it the column scan has a launch of
// its own (each block would read nb * E counts).
constexpr int kScanInBlocks = 128;

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

__global__ __launch_bounds__(kThreads) void block_hist_kernel(int n, int E, const int32_t* __restrict__ idx,
                                                              int32_t* __restrict__ hist) {
  __shared__ int32_t h[1024];
  for (int e = threadIdx.x; e < E; e += kThreads) h[e] = 0;
  __syncthreads();
  const int64_t f0 = static_cast<int64_t>(blockIdx.x) * kPermBlock;
  for (int i = threadIdx.x; i < kPermBlock; i += kThreads) {
    const int64_t f = f0 + i;
    if (f < n) atomicAdd(&h[clamp_expert(idx[f], E)], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) hist[static_cast<int64_t>(blockIdx.x) * E + e] = h[e];
}

// One block. Column scan of hist[nb][E] in place (exclusive: pairs of expert
// e in earlier blocks), counts[e] = column total, offsets = exclusive scan of
// counts.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(int nb, int E, int32_t* __restrict__ hist,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int32_t slab[kSlabInts];
  __shared__ int32_t part[kScanThreads];
  const int tid = threadIdx.x;
  const int rows_per_slab = kSlabInts / E;  // >= 8 since E <= 1024
  int32_t running = 0;                      // thread e < E owns column e
  for (int b0 = 0; b0 < nb; b0 += rows_per_slab) {
    const int rows = min(rows_per_slab, nb - b0);
    const int64_t base = static_cast<int64_t>(b0) * E;
    for (int q = tid; q < rows * E; q += kScanThreads) slab[q] = hist[base + q];
    __syncthreads();
    if (tid < E) {
      for (int r = 0; r < rows; ++r) {
        const int32_t c = slab[r * E + tid];
        slab[r * E + tid] = running;
        running += c;
      }
    }
    __syncthreads();
    for (int q = tid; q < rows * E; q += kScanThreads) hist[base + q] = slab[q];
    __syncthreads();
  }
  // Exclusive scan of the E column totals (Hillis-Steele over the block).
  part[tid] = tid < E ? running : 0;
  __syncthreads();
  for (int o = 1; o < kScanThreads; o <<= 1) {
    const int32_t v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  if (tid < E) {
    counts[tid] = running;
    offsets[tid] = part[tid] - running;
  }
  if (tid == E - 1) offsets[E] = part[tid];
}

constexpr int kWavesPerBlock = kThreads / kWave;

// The fused inference forward also takes, per sorted row p, its token
// row_token[p] = s2f[p] / k and its routing weight row_weight[p] = w[s2f[p]]
// (both null otherwise).
//
// SCAN = false: hist holds the column-scanned block counts and offsets is
// read (scan_kernel ran before). SCAN = true (few blocks): hist holds the raw
// block counts, and every block does the scan's work for itself instead of a
// launch of its own: the pairs of each expert in earlier blocks and in all
// blocks (nb reads per expert), then the exclusive scan of the totals over
// the experts; block 0 writes counts and offsets. Same integers either way.
template <bool SCAN>
__global__ __launch_bounds__(kThreads) void rank_scatter_kernel(int n, int E, int nbits,
                                                                const int32_t* __restrict__ idx,
                                                                const int32_t* __restrict__ hist_base,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ s2f,
                                                                int32_t* __restrict__ f2s, int k,
                                                                const float* __restrict__ w,
                                                                int32_t* __restrict__ row_token,
                                                                float* __restrict__ row_weight) {
  __shared__ int32_t running[1024];
  __shared__ int32_t wcount[kWavesPerBlock][1024];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wv = tid / kWave;
  if constexpr (SCAN) {
    __shared__ int32_t total[1024];
    __shared__ int32_t part[kWavesPerBlock];
    __shared__ int32_t pb[kThreads], pa[kThreads];
    const int nb = static_cast<int>(gridDim.x);
    const int blk = static_cast<int>(blockIdx.x);
    // Column sums with the block's G = 256 / E thread groups (one when E >
    // 256) each taking every G-th run of 32 blocks, 32 loads in flight.
    constexpr int kRun = 32;
    const int G = E <= kThreads ? kThreads / E : 1;
    const int g = tid / E;
    auto col = [&](int e, int32_t& before, int32_t& all) {
      before = 0;
      all = 0;
      for (int b0 = g * kRun; b0 < nb; b0 += G * kRun) {
        int32_t c[kRun];
#pragma unroll
        for (int u = 0; u < kRun; ++u) c[u] = b0 + u < nb ? hist_base[static_cast<int64_t>(b0 + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < kRun; ++u) {
          before += b0 + u < blk ? c[u] : 0;
          all += c[u];
        }
      }
    };
    if (G > 1) {
      int32_t before = 0, all = 0;
      if (g < G) col(tid % E, before, all);
      pb[tid] = before;
      pa[tid] = all;
      __syncthreads();
      for (int e = tid; e < E; e += kThreads) {
        int32_t sb = 0, sa = 0;
        for (int q = 0; q < G; ++q) {
          sb += pb[q * E + e];
          sa += pa[q * E + e];
        }
        running[e] = sb;
        total[e] = sa;
      }
    } else {
      for (int e = tid; e < E; e += kThreads) col(e, running[e], total[e]);
    }
    for (int e = tid; e < E; e += kThreads) {
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) wcount[w][e] = 0;
    }
    __syncthreads();
    // Exclusive scan of total[0..E): thread tid sums the run of `per`
    // experts starting at tid * per, a scan over the threads orders the
    // runs, and each run is then walked in expert order.
    const int per = (E + kThreads - 1) / kThreads;
    int32_t mine = 0;
    for (int q = 0; q < per; ++q) {
      const int e = tid * per + q;
      if (e < E) mine += total[e];
    }
    // inclusive scan of `mine` inside the wavefront, then across the four
    int32_t incl = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int32_t v = __shfl_up(incl, o);
      incl += lane >= o ? v : 0;
    }
    if (lane == kWave - 1) part[wv] = incl;
    __syncthreads();
    int32_t all_runs = 0;
#pragma unroll
    for (int q = 0; q < kWavesPerBlock; ++q) {
      incl += q < wv ? part[q] : 0;
      all_runs += part[q];
    }
    int32_t off = incl - mine;
    for (int q = 0; q < per; ++q) {
      const int e = tid * per + q;
      if (e < E) {
        running[e] += off;
        if (blk == 0) {
          counts[e] = total[e];
          offsets[e] = off;
        }
        off += total[e];
      }
    }
    if (blk == 0 && tid == 0) offsets[E] = all_runs;
  } else {
    for (int e = tid; e < E; e += kThreads) {
      running[e] = offsets[e] + hist_base[static_cast<int64_t>(blockIdx.x) * E + e];
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) wcount[w][e] = 0;
    }
  }
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t f0 = static_cast<int64_t>(blockIdx.x) * kPermBlock;
  for (int c0 = 0; c0 < kPermBlock; c0 += kThreads) {
    const int64_t f = f0 + c0 + tid;
    const bool valid = f < n;
    const int e = valid ? clamp_expert(idx[f], E) : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(valid && bit);
      peers &= bit ? ones : ~ones;
    }
    const int rank = __popcll(peers & below);
    if (valid && rank == 0) wcount[wv][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int32_t pos = running[e] + rank;
      for (int w = 0; w < wv; ++w) pos += wcount[w][e];
      s2f[pos] = static_cast<int32_t>(f);
      f2s[f] = pos;
      if (row_token) {
        row_token[pos] = static_cast<int32_t>(f / k);
        row_weight[pos] = w[f];
      }
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kThreads) {
      int32_t add = 0;
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) {
        add += wcount[w][ee];
        wcount[w][ee] = 0;
      }
      running[ee] += add;
    }
    __syncthreads();
  }
}

// x_perm[f2s[t k + j], :] = x[t, :] for j < k: one wavefront per token t.
// Each 16-byte chunk of the token's row is read once and written to the
// token's k sorted rows (a wavefront per sorted row would read every x row k
// times, in an order that misses the L2). The token index and its k
// destinations are wavefront-uniform.
__global__ __launch_bounds__(kThreads) void gather_kernel(int tokens, int k, int chunks_per_row,
                                                          const int32_t* __restrict__ f2s,
                                                          const uint4* __restrict__ x, uint4* __restrict__ x_perm) {
  const int lane = threadIdx.x % kWave;
  const int t = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kWavesPerBlock +
                                               static_cast<int>(threadIdx.x) / kWave);
  if (t >= tokens) return;
  const int64_t src = static_cast<int64_t>(t) * chunks_per_row;
  const int32_t* dst_rows = f2s + static_cast<int64_t>(t) * k;
  for (int c = lane; c < chunks_per_row; c += kWave) {
    const uint4 v = x[src + c];
    for (int j = 0; j < k; ++j) x_perm[static_cast<int64_t>(dst_rows[j]) * chunks_per_row + c] = v;
  }
}

}  // namespace

WsLayout ws_layout(const moe_shape& s) {
  WsLayout l{};
  const int64_t n = static_cast<int64_t>(s.T) * s.k;
  const int64_t nb = ceil_div64(n, kPermBlock);
  const size_t esz = s.dtype == MOE_BF16 ? 2 : 4;
  l.hist_off = 0;
  l.hist_bytes = static_cast<size_t>(nb) * s.E * sizeof(int32_t);
  l.dgu_off = (l.hist_bytes + 255) & ~static_cast<size_t>(255);
  l.dgu_bytes = static_cast<size_t>(n) * 2 * s.I * esz;
  l.part_off = (l.dgu_off + l.dgu_bytes + 255) & ~static_cast<size_t>(255);
  l.part_bytes = static_cast<size_t>(wgrad_part_tiles(s)) * 256 * 256 * sizeof(float);
  l.total = l.part_off + l.part_bytes;
  return l;
}

namespace {

// The stable counting sort shared by the permute entry points; hist holds
// ceil(T*k / kPermBlock) * E int32 (every element is written before it is read).
hipError_t launch_sort(const moe_shape& s, const int32_t* idx, int32_t* counts, int32_t* offsets, int32_t* s2f,
                       int32_t* f2s, const float* w, int32_t* row_token, float* row_weight, int32_t* hist,
                       hipStream_t st) {
  const int n = s.T * s.k;
  const int nb = ceil_div(n, kPermBlock);
  int nbits = 0;
  while ((1 << nbits) < s.E) ++nbits;
  block_hist_kernel<<<nb, kThreads, 0, st>>>(n, s.E, idx, hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (nb <= kScanInBlocks) {  // each ranking block scans for itself: one launch fewer
    rank_scatter_kernel<true><<<nb, kThreads, 0, st>>>(n, s.E, nbits, idx, hist, counts, offsets, s2f, f2s, s.k, w,
                                                       row_token, row_weight);
    return hipGetLastError();
  }
  scan_kernel<<<1, kScanThreads, 0, st>>>(nb, s.E, hist, counts, offsets);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  rank_scatter_kernel<false><<<nb, kThreads, 0, st>>>(n, s.E, nbits, idx, hist, counts, offsets, s2f, f2s, s.k, w,
                                                      row_token, row_weight);
  return hipGetLastError();
}

int32_t* ws_hist(const moe_shape& s, void* ws) {
  return reinterpret_cast<int32_t*>(static_cast<char*>(ws) + ws_layout(s).hist_off);
}

}  // namespace

hipError_t launch_permute(const moe_shape& s, const int32_t* idx, const void* x, int32_t* counts,
                          int32_t* offsets, int32_t* s2f, int32_t* f2s, void* x_perm, void* ws,
                          hipStream_t st) {
  hipError_t err = launch_sort(s, idx, counts, offsets, s2f, f2s, nullptr, nullptr, nullptr, ws_hist(s, ws), st);
  if (err != hipSuccess) return err;
  const int esz = s.dtype == MOE_BF16 ? 2 : 4;
  const int chunks = s.H * esz / 16;
  gather_kernel<<<ceil_div(s.T, kWavesPerBlock), kThreads, 0, st>>>(s.T, s.k, chunks, f2s,
                                                                    static_cast<const uint4*>(x),
                                                                    static_cast<uint4*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_permute_rows(const moe_shape& s, const int32_t* idx, const float* w, const void* x,
                               int32_t* counts, int32_t* offsets, int32_t* s2f, int32_t* f2s, int32_t* row_token,
                               float* row_weight, void* x_perm, void* ws, hipStream_t st) {
  hipError_t err = launch_sort(s, idx, counts, offsets, s2f, f2s, w, row_token, row_weight, ws_hist(s, ws), st);
  if (err != hipSuccess) return err;
  const int esz = s.dtype == MOE_BF16 ? 2 : 4;
  const int chunks = s.H * esz / 16;
  gather_kernel<<<ceil_div(s.T, kWavesPerBlock), kThreads, 0, st>>>(s.T, s.k, chunks, f2s,
                                                                    static_cast<const uint4*>(x),
                                                                    static_cast<uint4*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_permute_fused(const moe_shape& s, const int32_t* idx, const float* w, int32_t* counts,
                                int32_t* offsets, int32_t* s2f, int32_t* f2s, int32_t* row_token, float* row_weight,
                                void* ws, hipStream_t st) {
  return launch_sort(s, idx, counts, offsets, s2f, f2s, w, row_token, row_weight, ws_hist(s, ws), st);
}

size_t sort_hist_bytes(const moe_shape& s) { return ws_layout(s).hist_bytes; }

// The scratch array's address on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and kept.
hipError_t scratch_address(int32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    addr[dev] = p;
  }
  *out = static_cast<int32_t*>(addr[dev]);
  return hipSuccess;
}

hipError_t launch_permute_fused_noalloc(const moe_shape& s, const int32_t* idx, const float* w, int32_t* counts,
                                        int32_t* offsets, int32_t* s2f, int32_t* f2s, int32_t* row_token,
                                        float* row_weight, hipStream_t st) {
  int32_t* hist = nullptr;
  const hipError_t err = scratch_address(&hist);
  if (err != hipSuccess) return err;
  return launch_sort(s, idx, counts, offsets, s2f, f2s, w, row_token, row_weight, hist, st);
}

}  // namespace moe
