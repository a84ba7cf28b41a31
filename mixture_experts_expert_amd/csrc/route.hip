// Router kernels: logits, top-k + softmax + renormalisation, and the
// backward of the routing weights.
//
// The logits feed an integer decision (which experts a token goes to), so
// they are computed in a fixed order that a CPU can reproduce bit for bit: one
// fp32 fma chain per (token, expert) over h ascending from +0, then + bias.
// The chain runs on the vector ALUs; a matrix-core accumulation order is not
// specified and could not be matched. Each thread keeps 4 tokens x 2 experts
// = 8 independent chains in flight: per h it reads one float4 of tokens and
// one float2 of experts from LDS for 8 FMAs (3 bytes per FMA). A block covers
// 64 tokens x 32 experts, so that at T = 8192, E = 128 the grid gives every
// SIMD two wavefronts: with one, LDS returns at most about 120 bytes per clock
// and compute unit (the reads of one wavefront stay latency-bound), which
// caps the FMA rate at half the VALU's; with two it returns about 240, the
// 192 that the full FMA rate needs at 3 bytes per FMA.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRT = 4;              // tokens per thread
constexpr int kRE = 2;              // experts per thread
constexpr int kTy = 16, kTx = 16;   // thread grid of a block
constexpr int kTileT = kTy * kRT;   // 64 tokens per block
constexpr int kTileE = kTx * kRE;   // 32 experts per block
constexpr int kHC = 64;             // h values staged per step
constexpr int kLogitThreads = kTy * kTx;  // 256
constexpr int kXS = kTileT + 4;     // LDS row strides (floats), 16-byte aligned
constexpr int kWS = kTileE + 2;

// Staging of one kHC-wide h slice of `rows` rows into LDS as fp32 [h][row]:
// 16-byte global loads along h (coalesced), one thread per chunk.
template <class T, int ROWS>
struct Stager {
  static constexpr int VE = 16 / sizeof(T);            // elements per 16-byte chunk
  static constexpr int CPR = kHC / VE;                 // chunks per row
  static constexpr int PER = (ROWS * CPR + kLogitThreads - 1) / kLogitThreads;
  uint4 v[PER];
  __device__ __forceinline__ void load(const T* __restrict__ src, int row0, int nrows, int H, int h0, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + i * kLogitThreads;
      const int r = q / CPR, c = q % CPR;
      v[i] = make_uint4(0u, 0u, 0u, 0u);
      if (q < ROWS * CPR && row0 + r < nrows)
        v[i] = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(row0 + r) * H + h0 + c * VE);
    }
  }
  __device__ __forceinline__ void store(float* lds, int stride, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + i * kLogitThreads;
      if (q >= ROWS * CPR) continue;
      const int r = q / CPR, c = q % CPR;
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lds[(c * 8 + 2 * e) * stride + r] = __uint_as_float(w[e] << 16);
          lds[(c * 8 + 2 * e + 1) * stride + r] = __uint_as_float(w[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) lds[(c * 4 + e) * stride + r] = __uint_as_float(w[e]);
      }
    }
  }
};

template <class T>
__global__ __launch_bounds__(kLogitThreads) void router_logits_kernel(int Tn, int H, int E, const T* __restrict__ x,
                                                                      const T* __restrict__ wr,
                                                                      const float* __restrict__ bias,
                                                                      float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) float xs[2][kHC * kXS];  // [h][token]
  __shared__ __attribute__((aligned(16))) float ws[2][kHC * kWS];  // [h][expert]
  const int tid = threadIdx.x;
  const int ty = tid / kTx, tx = tid % kTx;
  const int t0 = blockIdx.x * kTileT;
  const int e0 = blockIdx.y * kTileE;

  float acc[kRT][kRE];
#pragma unroll
  for (int i = 0; i < kRT; ++i)
#pragma unroll
    for (int j = 0; j < kRE; ++j) acc[i][j] = 0.0f;

  Stager<T, kTileT> sx;
  Stager<T, kTileE> sw;
  sx.load(x, t0, Tn, H, 0, tid);
  sw.load(wr, e0, E, H, 0, tid);
  sx.store(xs[0], kXS, tid);
  sw.store(ws[0], kWS, tid);
  __syncthreads();
  const int nsteps = H / kHC;
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) {  // next slice in flight while this one is multiplied
      sx.load(x, t0, Tn, H, (s + 1) * kHC, tid);
      sw.load(wr, e0, E, H, (s + 1) * kHC, tid);
    }
    const float* xb = xs[buf];
    const float* wb = ws[buf];
#pragma unroll 16
    for (int hh = 0; hh < kHC; ++hh) {
      const float4 xv = *reinterpret_cast<const float4*>(xb + hh * kXS + ty * kRT);
      const float2 wv = *reinterpret_cast<const float2*>(wb + hh * kWS + tx * kRE);
      const float xa[kRT] = {xv.x, xv.y, xv.z, xv.w};
      const float wa[kRE] = {wv.x, wv.y};
#pragma unroll
      for (int i = 0; i < kRT; ++i)
#pragma unroll
        for (int j = 0; j < kRE; ++j) acc[i][j] = __fmaf_rn(xa[i], wa[j], acc[i][j]);
    }
    if (s + 1 < nsteps) {
      sx.store(xs[buf ^ 1], kXS, tid);
      sw.store(ws[buf ^ 1], kWS, tid);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < kRT; ++i) {
    const int t = t0 + ty * kRT + i;
    if (t >= Tn) continue;
    const int e = e0 + tx * kRE;
    float v[kRE];
#pragma unroll
    for (int j = 0; j < kRE; ++j) v[j] = (bias && e + j < E) ? acc[i][j] + bias[e + j] : acc[i][j];
    float* dst = logits + static_cast<int64_t>(t) * E + e;
    if (e + kRE <= E && (E % 2) == 0) {
      *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
    } else {
#pragma unroll
      for (int j = 0; j < kRE; ++j)
        if (e + j < E) dst[j] = v[j];
    }
  }
}

constexpr int kTokPerBlock = 4;  // one wave per token

// (value, index) order of the selection: larger value first, then lower
// index. A NaN ranks below every number, -inf included (two NaNs: the lower
// index first), so every token selects k valid experts whatever its logits.
__device__ __forceinline__ bool before(float v, int i, float ov, int oi) {
  const bool vn = v != v, on = ov != ov;
  if (vn != on) return on;
  return v > ov || (!(v < ov) && i < oi);
}

// NC logits per lane (E <= 64 NC): compiled per power of two up to 16, so
// that the selection loops run over the lane's own logits only.
template <int NC>
__global__ __launch_bounds__(kWave* kTokPerBlock) void router_topk_kernel(int Tn, int E, int k,
                                                                          const float* __restrict__ logits,
                                                                          int32_t* __restrict__ idx,
                                                                          float* __restrict__ w) {
  constexpr int kMaxPerLane = NC;
  __shared__ float sval[kTokPerBlock][1024];
  const int lane = threadIdx.x % kWave;
  const int wv = threadIdx.x / kWave;
  const int t = blockIdx.x * kTokPerBlock + wv;
  // Every wave runs to the block barrier below; a wave past the last token
  // works on -inf logits and stores nothing.
  const bool active = t < Tn;
  const float* l = logits + static_cast<int64_t>(active ? t : 0) * E;
  const int nc = (E + kWave - 1) / kWave;

  float v[kMaxPerLane];
  uint32_t valid = 0;  // bit c: v[c] holds a logit of this token
#pragma unroll
  for (int c = 0; c < kMaxPerLane; ++c) {
    const int e = lane + c * kWave;
    const bool in = active && c < nc && e < E;
    v[c] = in ? l[e] : -INFINITY;
    if (in) valid |= 1u << c;
  }
  uint32_t taken = ~valid;  // bit c: v[c] already selected (or not a logit)

  float vmax = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = __builtin_nanf("");  // below every candidate, NaN logits included
    int bi = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < kMaxPerLane; ++c) {
      if (taken & (1u << c)) continue;
      const int e = lane + c * kWave;
      if (before(v[c], e, bv, bi)) { bv = v[c]; bi = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (before(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (active && (bi % kWave) == lane) taken |= 1u << (bi / kWave);
    if (active && lane == 0) {
      idx[static_cast<int64_t>(t) * k + j] = bi;
      sval[wv][j] = bv;
    }
    if (j == 0) vmax = bv;
  }
  // Softmax denominator over all E logits, shifted by the maximum.
  float z = 0.0f;
#pragma unroll
  for (int c = 0; c < kMaxPerLane; ++c)
    if (valid & (1u << c)) z += expf(v[c] - vmax);
  z = wave_sum(z);
  __syncthreads();  // sval written by lane 0 becomes visible to its wave
  if (!active) return;
  float s = 0.0f;
  for (int j = lane; j < k; j += kWave) s += expf(sval[wv][j] - vmax) / z;
  s = wave_sum(s);
  const float den = s + 1e-20f;
  for (int j = lane; j < k; j += kWave)
    w[static_cast<int64_t>(t) * k + j] = (expf(sval[wv][j] - vmax) / z) / den;
}

__global__ __launch_bounds__(kWave* kTokPerBlock) void router_bwd_kernel(int Tn, int E, int k,
                                                                         const float* __restrict__ gw,
                                                                         const float* __restrict__ w,
                                                                         const int32_t* __restrict__ idx,
                                                                         float* __restrict__ d_logits) {
  __shared__ float row[kTokPerBlock][1024];
  const int lane = threadIdx.x % kWave;
  const int wv = threadIdx.x / kWave;
  const int t = blockIdx.x * kTokPerBlock + wv;
  const bool active = t < Tn;
  const int64_t tk = static_cast<int64_t>(t) * k;
  float gs = 0.0f;
  if (active) {
    for (int j = lane; j < k; j += kWave) gs += w[tk + j] * gw[tk + j];
    for (int e = lane; e < E; e += kWave) row[wv][e] = 0.0f;
  }
  gs = wave_sum(gs);
  __syncthreads();
  if (active)
    for (int j = lane; j < k; j += kWave) {
      const int e = idx[tk + j];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) row[wv][e] = w[tk + j] * (gw[tk + j] - gs);
    }
  __syncthreads();
  if (active)
    for (int e = lane; e < E; e += kWave) d_logits[static_cast<int64_t>(t) * E + e] = row[wv][e];
}

}  // namespace

hipError_t launch_route(const moe_shape& s, const void* x, const void* wr, const float* bias, float* logits,
                        int32_t* idx, float* w, hipStream_t st) {
  dim3 grid(ceil_div(s.T, kTileT), ceil_div(s.E, kTileE));
  if (s.dtype == MOE_BF16)
    router_logits_kernel<bf16_t><<<grid, kLogitThreads, 0, st>>>(
        s.T, s.H, s.E, static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(wr), bias, logits);
  else
    router_logits_kernel<float><<<grid, kLogitThreads, 0, st>>>(
        s.T, s.H, s.E, static_cast<const float*>(x), static_cast<const float*>(wr), bias, logits);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 g(ceil_div(s.T, kTokPerBlock)), b(kWave * kTokPerBlock);
  const int nc = ceil_div(s.E, kWave);
  if (nc <= 1) router_topk_kernel<1><<<g, b, 0, st>>>(s.T, s.E, s.k, logits, idx, w);
  else if (nc <= 2) router_topk_kernel<2><<<g, b, 0, st>>>(s.T, s.E, s.k, logits, idx, w);
  else if (nc <= 4) router_topk_kernel<4><<<g, b, 0, st>>>(s.T, s.E, s.k, logits, idx, w);
  else if (nc <= 8) router_topk_kernel<8><<<g, b, 0, st>>>(s.T, s.E, s.k, logits, idx, w);
  else router_topk_kernel<16><<<g, b, 0, st>>>(s.T, s.E, s.k, logits, idx, w);
  return hipGetLastError();
}

hipError_t launch_route_bwd(const moe_shape& s, const float* gw, const float* w, const int32_t* idx,
                            float* d_logits, hipStream_t st) {
  router_bwd_kernel<<<ceil_div(s.T, kTokPerBlock), kWave * kTokPerBlock, 0, st>>>(s.T, s.E, s.k, gw, w, idx,
                                                                                   d_logits);
  return hipGetLastError();
}

}  // namespace moe
