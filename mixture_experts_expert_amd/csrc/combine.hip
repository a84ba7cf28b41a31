// Weighted combine (forward), its backward, and the unpermute-sum.
//
// The combine follows modelopt.torch.utils.moe, a2a_moe: a token's k expert
// results are weighted by its routing weights in the weights' own precision
// (fp32 here) and summed, then returned in the hidden dtype. One wavefront
// handles one token; each lane owns 16-byte column chunks, so every row read
// and the output row write are contiguous across the wavefront, and a
// token's rows are read in batches so that several are in flight at once.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

template <class T> struct Vec;
template <> struct Vec<float> {
  static constexpr int N = 4;  // elements per 16-byte chunk
  __device__ __forceinline__ static void unpack(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static uint4 pack(const float* o) {
    return make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3]));
  }
};
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const uint4& v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static uint4 pack(const float* o) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// Rows of one token in flight together: a batch's row indices (and weights)
// come in with one vector load (lane j holds slot j) and are broadcast with
// readlane, then every row's chunk is loaded, then the sums run in slot
// order. Slots past k reload the last row and are masked out of the sum
// (a select, not a branch, so that no load sinks into a conditional).
constexpr int kBatch = 8;

// Slot j0 + lane's row index and weight (lanes >= kBatch and slots past k
// repeat the last slot); broadcast one of them with slot_bcast.
__device__ __forceinline__ void load_slots(const int32_t* __restrict__ f2s, const float* __restrict__ w,
                                           int64_t tk, int j0, int k, int lane, int& idx, float& wt) {
  const int j = min(j0 + min(lane, kBatch - 1), k - 1);
  idx = f2s[tk + j];
  wt = w ? w[tk + j] : 1.0f;
}
__device__ __forceinline__ int slot_bcast(int v, int jj) { return __builtin_amdgcn_readlane(v, jj); }
__device__ __forceinline__ float slot_bcast(float v, int jj) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), jj));
}

// y[t] = sum_j w[t,j] * o_perm[f2s[t*k+j]]   (WEIGHTED)   or   sum_j src[f2s[t*k+j]]
// fp32 sums in ascending j, one rounding to T at the end.
template <class T, bool WEIGHTED>
__global__ __launch_bounds__(kThreads) void gather_sum_kernel(int Tn, int k, int chunks,
                                                              const uint4* __restrict__ src,
                                                              const float* __restrict__ w,
                                                              const int32_t* __restrict__ f2s,
                                                              uint4* __restrict__ out) {
  constexpr int N = Vec<T>::N;
  const int lane = threadIdx.x % kWave;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock + static_cast<int>(threadIdx.x) / kWave);
  if (t >= Tn) return;
  const int64_t tk = static_cast<int64_t>(t) * k;
  if (k <= kBatch) {
    // One batch of slots: the row indices once, then two bands of 64 chunks
    // (16 row chunks) in flight together. A second band past the row repeats
    // the first band's chunk and stores the same bytes there again (no branch
    // for the loads to sink into).
    int idx;
    float wt;
    load_slots(f2s, WEIGHTED ? w : nullptr, tk, 0, k, lane, idx, wt);
    int64_t row[kBatch];
    float wj[kBatch];
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      row[jj] = static_cast<int64_t>(slot_bcast(idx, jj)) * chunks;
      wj[jj] = slot_bcast(wt, jj);
    }
    for (int c = lane; c < chunks; c += 2 * kWave) {
      const bool second = c + kWave < chunks;
      const int c2 = second ? c + kWave : c;
      uint4 v[2][kBatch];
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) {
        v[0][jj] = src[row[jj] + c];
        v[1][jj] = src[row[jj] + c2];
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float acc[N];
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int jj = 0; jj < kBatch; ++jj) {
          const bool live = jj < k;
          float x[N];
          Vec<T>::unpack(v[b][jj], x);
#pragma unroll
          for (int i = 0; i < N; ++i) {
            const float sum = WEIGHTED ? acc[i] + wj[jj] * x[i] : acc[i] + x[i];
            acc[i] = live ? sum : acc[i];
          }
        }
        out[static_cast<int64_t>(t) * chunks + (b == 0 ? c : c2)] = Vec<T>::pack(acc);
      }
    }
    return;
  }
  for (int c = lane; c < chunks; c += kWave) {
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += kBatch) {
      int idx;
      float wt;
      load_slots(f2s, WEIGHTED ? w : nullptr, tk, j0, k, lane, idx, wt);
      uint4 v[kBatch];
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) v[jj] = src[static_cast<int64_t>(slot_bcast(idx, jj)) * chunks + c];
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) {
        const bool live = j0 + jj < k;
        const float wj = slot_bcast(wt, jj);
        float x[N];
        Vec<T>::unpack(v[jj], x);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const float sum = WEIGHTED ? acc[i] + wj * x[i] : acc[i] + x[i];
          acc[i] = live ? sum : acc[i];
        }
      }
    }
    out[static_cast<int64_t>(t) * chunks + c] = Vec<T>::pack(acc);
  }
}

// do_perm[p] = w[t,j] * dy[t];  gw[t,j] = <dy[t], o_perm[p]>,  p = f2s[t*k+j]
// Slots go in batches of BATCH; for each batch the row is walked in bands of
// kWave chunks with the batch's o_perm chunks in flight together. Without
// do_perm (WRITE_DO false: the backward that reads dy through the rows'
// tokens) only gw is written, eight slots at a time.
template <class T, bool WRITE_DO, int BATCH>
__global__ __launch_bounds__(kThreads) void combine_bwd_kernel(int Tn, int k, int chunks,
                                                               const uint4* __restrict__ dy,
                                                               const uint4* __restrict__ o_perm,
                                                               const float* __restrict__ w,
                                                               const int32_t* __restrict__ f2s,
                                                               uint4* __restrict__ do_perm,
                                                               float* __restrict__ gw) {
  constexpr int N = Vec<T>::N;
  const int lane = threadIdx.x % kWave;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock + static_cast<int>(threadIdx.x) / kWave);
  if (t >= Tn) return;  // wave-uniform: no block barrier in this kernel
  const int64_t tk = static_cast<int64_t>(t) * k;
  constexpr int kBwdBatch = BATCH;
  for (int j0 = 0; j0 < k; j0 += kBwdBatch) {
    int idx;
    float wt;
    load_slots(f2s, w, tk, j0, k, lane, idx, wt);
    int64_t p[kBwdBatch];
    float wj[kBwdBatch], dot[kBwdBatch];
#pragma unroll
    for (int jj = 0; jj < kBwdBatch; ++jj) {
      p[jj] = slot_bcast(idx, jj);
      wj[jj] = slot_bcast(wt, jj);
      dot[jj] = 0.0f;
    }
    for (int c = lane; c < chunks; c += kWave) {
      const uint4 dv = dy[static_cast<int64_t>(t) * chunks + c];
      uint4 ov[kBwdBatch];
#pragma unroll
      for (int jj = 0; jj < kBwdBatch; ++jj) ov[jj] = o_perm[p[jj] * chunks + c];
      float d[N];
      Vec<T>::unpack(dv, d);
#pragma unroll
      for (int jj = 0; jj < kBwdBatch; ++jj) {
        float o[N], g[N];
        Vec<T>::unpack(ov[jj], o);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          g[i] = wj[jj] * d[i];
          dot[jj] += d[i] * o[i];
        }
        // Slots past k repeat the last row: the same values again, harmless.
        if constexpr (WRITE_DO) do_perm[p[jj] * chunks + c] = Vec<T>::pack(g);
      }
    }
#pragma unroll
    for (int jj = 0; jj < kBwdBatch; ++jj) {
      if (j0 + jj >= k) break;
      const float sdot = wave_sum(dot[jj]);
      if (lane == 0) gw[tk + j0 + jj] = sdot;
    }
  }
}

template <class T, bool WEIGHTED>
hipError_t gather_sum(const moe_shape& s, const void* src, const float* w, const int32_t* f2s, void* out,
                      hipStream_t st) {
  const int chunks = s.H / Vec<T>::N;
  gather_sum_kernel<T, WEIGHTED><<<ceil_div(s.T, kWavesPerBlock), kThreads, 0, st>>>(
      s.T, s.k, chunks, static_cast<const uint4*>(src), w, f2s, static_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const moe_shape& s, const void* o_perm, const float* w, const int32_t* f2s, void* y,
                          hipStream_t st) {
  return s.dtype == MOE_BF16 ? gather_sum<bf16_t, true>(s, o_perm, w, f2s, y, st)
                             : gather_sum<float, true>(s, o_perm, w, f2s, y, st);
}

hipError_t launch_unpermute_sum(const moe_shape& s, const void* dx_perm, const int32_t* f2s, void* dx,
                                hipStream_t st) {
  return s.dtype == MOE_BF16 ? gather_sum<bf16_t, false>(s, dx_perm, nullptr, f2s, dx, st)
                             : gather_sum<float, false>(s, dx_perm, nullptr, f2s, dx, st);
}

hipError_t launch_combine_bwd(const moe_shape& s, const void* dy, const void* o_perm, const float* w,
                              const int32_t* f2s, void* do_perm, float* gw, hipStream_t st) {
  const dim3 grid(ceil_div(s.T, kWavesPerBlock));
  const uint4* d = static_cast<const uint4*>(dy);
  const uint4* o = static_cast<const uint4*>(o_perm);
  uint4* dp = static_cast<uint4*>(do_perm);
  if (s.dtype == MOE_BF16) {
    const int ch = s.H / Vec<bf16_t>::N;
    if (do_perm) combine_bwd_kernel<bf16_t, true, 4><<<grid, kThreads, 0, st>>>(s.T, s.k, ch, d, o, w, f2s, dp, gw);
    else combine_bwd_kernel<bf16_t, false, 8><<<grid, kThreads, 0, st>>>(s.T, s.k, ch, d, o, w, f2s, dp, gw);
  } else {
    const int ch = s.H / Vec<float>::N;
    if (do_perm) combine_bwd_kernel<float, true, 4><<<grid, kThreads, 0, st>>>(s.T, s.k, ch, d, o, w, f2s, dp, gw);
    else combine_bwd_kernel<float, false, 8><<<grid, kThreads, 0, st>>>(s.T, s.k, ch, d, o, w, f2s, dp, gw);
  }
  return hipGetLastError();
}

}  // namespace moe
