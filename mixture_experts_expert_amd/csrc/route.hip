// Router kernels: logits, top-k + softmax + renormalisation, and the
// backward of the routing weights.
//
// The logits feed an integer decision (which experts a token goes to), so
// they are computed in a fixed order that a CPU can reproduce bit for bit: one
// fp32 fma chain per (token, expert) over h ascending from +0, then + bias.
// The chain runs on the vector ALUs; a matrix-core accumulation order is not
// specified and could not be matched.
//
// A lane owns one token and eight chains (eight experts). Its token's x comes
// from LDS (4 bytes per h for 8 FMAs); the experts' weights are wavefront-
// uniform, and a DPP row broadcast supplies them as the first operand of
// v_fmac_f32 itself: lane n of each 16-lane row holds w[e_(n%8)][h] for the
// eight h of one half of a 16-h batch, and `row_newbcast:n` hands that value
// to every lane of the row. A batch of 16 h costs each lane 6 LDS reads of 16
// bytes for 128 FMAs (0.75 byte per FMA), so the FMAs, not LDS, set the pace.
// A block covers 64 tokens x 32 experts (four wavefronts of eight experts);
// at T = 8192, E = 128 the grid gives every SIMD two wavefronts.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kEW = 8;                     // experts per wavefront (chains per lane)
constexpr int kLogitWaves = 4;
constexpr int kTileT = kWave;              // 64 tokens per block, one per lane
constexpr int kTileE = kLogitWaves * kEW;  // 32 experts per block
constexpr int kHC = 64;                    // h values staged per LDS slice
constexpr int kHB = 16;                    // h values per register batch
constexpr int kLogitThreads = kLogitWaves * kWave;  // 256
constexpr int kRS = kHC + 4;               // LDS row stride (floats): 16-byte aligned, rows 4 banks apart

// Staging of one kHC-wide h slice of `ROWS` rows into LDS as fp32 [row][h]:
// 16-byte global loads along h (coalesced), one thread per chunk; rows past
// `nrows` are zero.
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
  __device__ __forceinline__ void store(float* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + i * kLogitThreads;
      if (q >= ROWS * CPR) continue;
      const int r = q / CPR, c = q % CPR;
      float* dst = lds + r * kRS + c * VE;
      if constexpr (sizeof(T) == 2) {
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = __uint_as_float(w[e] << 16);
          f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
        reinterpret_cast<float4*>(dst)[0] = make_float4(f[0], f[1], f[2], f[3]);
        reinterpret_cast<float4*>(dst)[1] = make_float4(f[4], f[5], f[6], f[7]);
      } else {
        *reinterpret_cast<float4*>(dst) =
            make_float4(__uint_as_float(v[i].x), __uint_as_float(v[i].y), __uint_as_float(v[i].z),
                        __uint_as_float(v[i].w));
      }
    }
  }
};

// Eight h steps of the eight chains: for k = 0..7 and j = 0..7,
// a[j] = fma(w_j(h_k), x[k], a[j]), where w_j(h_k) is register w[k] of lane
// L0 + j of the row (DPP row_newbcast). The chains advance h by h, so each
// stays in h order. The leading s_nop keeps two wait states between a VALU
// write of a broadcast source and its DPP read.
#define RB_F(A, W, X, L) "v_fmac_f32_dpp %" #A ", %" #W ", %" #X " row_newbcast:" #L " row_mask:0xf bank_mask:0xf\n"
#define RB_K(W, X, L0, L1, L2, L3, L4, L5, L6, L7)                                                          \
  RB_F(0, W, X, L0) RB_F(1, W, X, L1) RB_F(2, W, X, L2) RB_F(3, W, X, L3) RB_F(4, W, X, L4) RB_F(5, W, X, L5) \
  RB_F(6, W, X, L6) RB_F(7, W, X, L7)
#define RB_HALF(...)                                                                                    \
  "s_nop 1\n" RB_K(8, 16, __VA_ARGS__) RB_K(9, 17, __VA_ARGS__) RB_K(10, 18, __VA_ARGS__)             \
      RB_K(11, 19, __VA_ARGS__) RB_K(12, 20, __VA_ARGS__) RB_K(13, 21, __VA_ARGS__) RB_K(14, 22, __VA_ARGS__) \
          RB_K(15, 23, __VA_ARGS__)
#define RB_OPERANDS                                                                                        \
  : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])        \
  : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]), "v"(x[0]),    \
    "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7])

template <int HALF>
__device__ __forceinline__ void fma_8h(float (&a)[kEW], const float (&w)[8], const float* x) {
  if constexpr (HALF == 0)
    asm(RB_HALF(0, 1, 2, 3, 4, 5, 6, 7) RB_OPERANDS);
  else
    asm(RB_HALF(8, 9, 10, 11, 12, 13, 14, 15) RB_OPERANDS);
}
#undef RB_F
#undef RB_K
#undef RB_HALF
#undef RB_OPERANDS

template <class T>
__global__ __launch_bounds__(kLogitThreads) void router_logits_kernel(int Tn, int H, int E, const T* __restrict__ x,
                                                                      const T* __restrict__ wr,
                                                                      const float* __restrict__ bias,
                                                                      float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) float xs[2][kTileT * kRS];  // [token][h]
  __shared__ __attribute__((aligned(16))) float ws[2][kTileE * kRS];  // [expert][h]
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int n = lane % 16;  // lane within its DPP row
  const int t0 = blockIdx.x * kTileT;
  const int e0 = blockIdx.y * kTileE;

  float acc[kEW];
#pragma unroll
  for (int j = 0; j < kEW; ++j) acc[j] = 0.0f;
  // This wavefront's experts and their biases, loaded now so that their
  // latency hides behind the chains.
  const int e = e0 + wave * kEW;
  float bv[kEW];
#pragma unroll
  for (int j = 0; j < kEW; ++j) bv[j] = (bias && e + j < E) ? bias[e + j] : 0.0f;

  Stager<T, kTileT> sx;
  Stager<T, kTileE> sw;
  sx.load(x, t0, Tn, H, 0, tid);
  sw.load(wr, e0, E, H, 0, tid);
  sx.store(xs[0], tid);
  sw.store(ws[0], tid);
  __syncthreads();
  // This lane's broadcast slots: expert e0 + 8 wave + n % 8, the half n / 8 of
  // each 16-h batch.
  const int xoff = lane * kRS;
  const int woff = (wave * kEW + (n & 7)) * kRS + (n >> 3) * 8;
  const int nsteps = H / kHC;
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) {  // next slice in flight while this one is multiplied
      sx.load(x, t0, Tn, H, (s + 1) * kHC, tid);
      sw.load(wr, e0, E, H, (s + 1) * kHC, tid);
    }
    const float* xb = xs[buf] + xoff;
    const float* wb = ws[buf] + woff;
    // Batch b + 1's LDS reads are in flight while batch b's FMAs run.
    float xv[2][kHB], wv[2][8];
    auto read_batch = [&](int hb, float(&xr)[kHB], float(&wr8)[8]) {
#pragma unroll
      for (int i = 0; i < kHB / 4; ++i) {
        const float4 q = *reinterpret_cast<const float4*>(xb + hb + 4 * i);
        xr[4 * i] = q.x;
        xr[4 * i + 1] = q.y;
        xr[4 * i + 2] = q.z;
        xr[4 * i + 3] = q.w;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float4 q = *reinterpret_cast<const float4*>(wb + hb + 4 * i);
        wr8[4 * i] = q.x;
        wr8[4 * i + 1] = q.y;
        wr8[4 * i + 2] = q.z;
        wr8[4 * i + 3] = q.w;
      }
    };
    read_batch(0, xv[0], wv[0]);
#pragma unroll
    for (int b = 0; b < kHC / kHB; ++b) {
      if (b + 1 < kHC / kHB) read_batch((b + 1) * kHB, xv[(b + 1) & 1], wv[(b + 1) & 1]);
      fma_8h<0>(acc, wv[b & 1], xv[b & 1]);
      fma_8h<1>(acc, wv[b & 1], xv[b & 1] + 8);
    }
    if (s + 1 < nsteps) {
      sx.store(xs[buf ^ 1], tid);
      sw.store(ws[buf ^ 1], tid);
    }
    __syncthreads();
  }

  const int t = t0 + lane;
  if (t >= Tn) return;
  float v[kEW];
#pragma unroll
  for (int j = 0; j < kEW; ++j) v[j] = bias ? acc[j] + bv[j] : acc[j];
  float* dst = logits + static_cast<int64_t>(t) * E + e;
  if (e + kEW <= E && (E % 4) == 0) {
    reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
#pragma unroll
    for (int j = 0; j < kEW; ++j)
      if (e + j < E) dst[j] = v[j];
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

// The top-k for E <= 256 and k <= 16: one token per 16-lane DPP row (four
// per wavefront), NC logits per lane (e = n + 16 c), every cross-lane step a
// DPP move. A selection key orders (logit, index) as `before` does: the
// logit's order bits (NaN lowest; -0 counted as +0, so equal logits tie on the
// index) above the complement of the index. Taken and absent slots hold 0,
// below every key, so one unsigned max per round picks the next expert.
constexpr int kRowTopkThreads = 256;
constexpr int kRowTok = kRowTopkThreads / 16;  // tokens per block

__device__ __forceinline__ uint64_t sel_key(float v, int e) {
  const float c = v + 0.0f;  // -0 -> +0
  const uint32_t b = __float_as_uint(c);
  const uint32_t o = (c != c) ? 0u : ((b & 0x80000000u) ? ~b : (b | 0x80000000u));
  return (static_cast<uint64_t>(o) << 32) | static_cast<uint32_t>(~e);
}

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t o = static_cast<uint32_t>(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);  // o = 0: a NaN
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// Quad swaps (quad_perm [1,0,3,2] and [2,3,0,1]), then half-row and row
// mirrors: every lane of a 16-lane row ends with the row's maximum (or sum).
__device__ __forceinline__ uint64_t row_max_key(uint64_t k) {
#define RM_STEP(CTRL)                                                                                      \
  {                                                                                                        \
    const uint64_t o = (static_cast<uint64_t>(dpp32<CTRL>(static_cast<uint32_t>(k >> 32))) << 32) |       \
                       dpp32<CTRL>(static_cast<uint32_t>(k));                                              \
    k = o > k ? o : k;                                                                                     \
  }
  RM_STEP(0xB1) RM_STEP(0x4E) RM_STEP(0x141) RM_STEP(0x140)
#undef RM_STEP
  return k;
}

__device__ __forceinline__ float row_sum(float v) {
  v += __uint_as_float(dpp32<0xB1>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<0x4E>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<0x141>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<0x140>(__float_as_uint(v)));
  return v;
}

template <int NC>
__global__ __launch_bounds__(kRowTopkThreads) void router_topk_row_kernel(int Tn, int E, int k,
                                                                         const float* __restrict__ logits,
                                                                         int32_t* __restrict__ idx,
                                                                         float* __restrict__ w) {
  const int n = threadIdx.x % 16;
  const int t = blockIdx.x * kRowTok + threadIdx.x / 16;
  // A row past the last token runs on absent slots (every DPP step needs all
  // lanes) and stores nothing.
  const bool active = t < Tn;
  const float* l = logits + static_cast<int64_t>(active ? t : 0) * E;
  float v[NC];
  uint64_t key[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int e = n + 16 * c;
    const bool in = active && e < E;
    v[c] = in ? l[e] : 0.0f;
    key[c] = in ? sel_key(v[c], e) : 0;
  }
  float sel_v = 0.0f, vmax = 0.0f;  // round j's logit and expert, kept by lane j
  int sel_i = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t b = key[0];
#pragma unroll
    for (int c = 1; c < NC; ++c) b = key[c] > b ? key[c] : b;
    b = row_max_key(b);
    const float bv = key_value(b);
    if (j == 0) vmax = bv;
    if (n == j) {
      sel_v = bv;
      sel_i = static_cast<int>(~static_cast<uint32_t>(b));
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) key[c] = key[c] == b ? 0 : key[c];  // keys are unique
  }
  // Softmax denominator over all E logits, shifted by the maximum.
  float z = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (active && n + 16 * c < E) z += expf(v[c] - vmax);
  z = row_sum(z);
  const float p = n < k ? expf(sel_v - vmax) / z : 0.0f;
  const float den = row_sum(p) + 1e-20f;
  if (active && n < k) {
    idx[static_cast<int64_t>(t) * k + n] = sel_i;
    w[static_cast<int64_t>(t) * k + n] = p / den;
  }
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
  if (s.E <= 256 && s.k <= 16) {
    const dim3 g(ceil_div(s.T, kRowTok)), b(kRowTopkThreads);
    const int nc = ceil_div(s.E, 16);
    if (nc <= 1) router_topk_row_kernel<1><<<g, b, 0, st>>>(s.T, s.E, s.k, logits, idx, w);
    else if (nc <= 2) router_topk_row_kernel<2><<<g, b, 0, st>>>(s.T, s.E, s.k, logits, idx, w);
    else if (nc <= 4) router_topk_row_kernel<4><<<g, b, 0, st>>>(s.T, s.E, s.k, logits, idx, w);
    else if (nc <= 8) router_topk_row_kernel<8><<<g, b, 0, st>>>(s.T, s.E, s.k, logits, idx, w);
    else router_topk_row_kernel<16><<<g, b, 0, st>>>(s.T, s.E, s.k, logits, idx, w);
    return hipGetLastError();
  }
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
