// Rows of a bf16 matrix -> 4-bit floats in the OCP microscaling FP4 format
// (MXFP4), for adapters over 4-bit frozen experts.
//
// The pages train adapters over 4-bit frozen weights (sourcepulse summary,
// "Highlighted Details": QLoRA on the fused experts; "Quick Start &
// Requirements": bitsandbytes 4-bit weights). Elements are E2M1 (sign, 2
// exponent bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2,
// 3, 4, 6); every 32 consecutive elements of a row share a power-of-two
// scale, stored as a biased exponent byte (E8M0, 2^(c - 127)): the smallest
// X with max |block| / 2^X <= 6, so nothing is clipped. Dividing by 2^X is
// exact; the element is then rounded to the nearest E2M1 magnitude, ties to
// the even mantissa, and keeps its sign. Two elements per byte, the even one
// in the low nibble.
//
// One thread per block of 32: four 16-byte loads, one 16-byte store of the
// codes and one byte of scale; neighbouring threads take neighbouring blocks.
// The scales are stored row-major ([rows][K/32], for the adapter merge) or,
// for the MXFP4 GEMMs, block-major within each expert's rows ([E][K/32][N]),
// so that one k-step's scales of consecutive weight rows are contiguous.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// E2M1 magnitude code of a in [0, 6]: the number of midpoints between
// neighbouring magnitudes that a lies above, a midpoint that a equals
// counting when it rounds up to the even code (1 -> 2, 3 -> 4, 5 -> 6).
__device__ __forceinline__ uint32_t e2m1_code(float a) {
  return static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) + static_cast<uint32_t>(a > 1.25f) +
         static_cast<uint32_t>(a >= 1.75f) + static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
         static_cast<uint32_t>(a > 5.0f);
}

__global__ __launch_bounds__(kThreads) void quantize_mxfp4_kernel(int64_t blocks, int kb, int kmajor_rows,
                                                                  const uint4* __restrict__ in,
                                                                  uint4* __restrict__ q, uint8_t* __restrict__ e8) {
  const int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (b >= blocks) return;
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = in[4 * b + i];
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
  float v[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int X = -127;
  if (amax > 0.0f) {
    // amax = f 2^ex, f in [0.5, 1); 6 = 0.75 2^3, so amax / 2^(ex - 3) = 8 f
    // is at most 6 exactly when f <= 0.75, else one power more.
    int ex;
    const float f = frexpf(amax, &ex);
    X = min(127, max(-127, ex - 3 + (f > 0.75f ? 1 : 0)));
  }
  uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t sign = (__float_as_uint(v[i]) >> 31) << 3;
    const uint32_t code = e2m1_code(fabsf(ldexpf(v[i], -X))) | sign;
    packed[i >> 3] |= code << (4 * (i & 7));
  }
  q[b] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  int64_t si = b;  // scale of block j of row `row`: [rows][kb], or [group][kb][R] with R = kmajor_rows
  if (kmajor_rows > 0) {
    const int64_t row = b / kb, j = b - row * kb;
    si = (row / kmajor_rows) * kb * kmajor_rows + j * kmajor_rows + row % kmajor_rows;
  }
  e8[si] = static_cast<uint8_t>(X + 127);
}

}  // namespace

hipError_t launch_quantize_mxfp4_rows(int rows, int K, const void* in, uint8_t* q, uint8_t* e8, int kmajor_rows,
                                      hipStream_t st) {
  const int64_t blocks = static_cast<int64_t>(rows) * (K / 32);
  if (blocks == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((blocks + kThreads - 1) / kThreads);
  quantize_mxfp4_kernel<<<grid, kThreads, 0, st>>>(blocks, K / 32, kmajor_rows, static_cast<const uint4*>(in),
                                                   reinterpret_cast<uint4*>(q), e8);
  return hipGetLastError();
}

}  // namespace moe
