// Rows of a bf16 matrix -> 8-bit floats (OCP E4M3) with one power-of-two
// scale per row, for the fp8 expert GEMMs.
//
// The pages' memory-saving path keeps expert weights in fewer bits
// (sourcepulse summary: bitsandbytes 4-bit weights, "Quick Start &
// Requirements"; QLoRA and quantised GGUF models, "Highlighted Details").
// Here both GEMM operands are E4M3 and each row carries its scale as a
// biased exponent byte (E8M0, 2^(c - 127)): the smallest X with
// max |x| / 2^X <= 448, so the row's largest element lands in (224, 448] and
// nothing is clipped. Dividing by 2^X is exact, so the only rounding is the
// conversion to E4M3 (nearest, ties to even), which the hardware does; the
// clamp to +-448 before it (a no-op unless X hit its limit of 127) is there
// because the conversion turns values past 448 into NaN instead of
// saturating.
//
// One wavefront per row; lanes take 16-byte chunks (8 elements) of it.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kWave;

__device__ __forceinline__ void unpack8(const uint4& v, float* o) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(int rows, int K, const uint4* __restrict__ in,
                                                                 uint2* __restrict__ q, uint8_t* __restrict__ e8,
                                                                 const int32_t* __restrict__ flat_to_sorted, int k) {
  const int row = blockIdx.x * kRowsPerBlock + static_cast<int>(threadIdx.x) / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= rows) return;
  const int chunks = K / 8;
  const uint4* src = in + static_cast<int64_t>(row) * chunks;
  float amax = 0.0f;
  for (int c = lane; c < chunks; c += kWave) {
    float v[8];
    unpack8(src[c], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  int X = -127;
  if (amax > 0.0f) {
    // amax = f 2^ex, f in [0.5, 1); 448 = 0.875 2^9, so amax / 2^(ex - 9) =
    // 512 f is at most 448 exactly when f <= 0.875, else one power more.
    int ex;
    const float f = frexpf(amax, &ex);
    X = min(127, max(-127, ex - 9 + (f > 0.875f ? 1 : 0)));
  }
  uint2* dst = q + static_cast<int64_t>(row) * chunks;
  for (int c = lane; c < chunks; c += kWave) {
    float v[8];
    unpack8(src[c], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fminf(fmaxf(ldexpf(v[i], -X), -448.0f), 448.0f);
    int lo = 0, hi = 0;
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], lo, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], hi, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], hi, true);
    dst[c] = make_uint2(static_cast<uint32_t>(lo), static_cast<uint32_t>(hi));
  }
  const uint8_t code = static_cast<uint8_t>(X + 127);
  if (flat_to_sorted == nullptr) {
    if (lane == 0) e8[row] = code;
  } else {  // a token's scale at each of its k sorted rows
    for (int j = lane; j < k; j += kWave) e8[flat_to_sorted[static_cast<int64_t>(row) * k + j]] = code;
  }
}

}  // namespace

hipError_t launch_quantize_fp8_rows(int rows, int K, const void* in, uint8_t* q, uint8_t* e8,
                                    const int32_t* flat_to_sorted, int k, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  quantize_rows_kernel<<<blocks, kThreads, 0, st>>>(rows, K, static_cast<const uint4*>(in),
                                                    reinterpret_cast<uint2*>(q), e8, flat_to_sorted, k);
  return hipGetLastError();
}

}  // namespace moe
