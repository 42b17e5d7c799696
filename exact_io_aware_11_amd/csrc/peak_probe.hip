// Matrix-core rate probe: a pure stream of 32x32 MFMAs (bf16 32x32x16 or
// fp8 32x32x64) on fixed pseudo-random per-lane operands, two waves per SIMD
// on every CU.  It measures what the matrix cores sustain on this chip with
// data whose bits toggle like real inputs -- the chip lowers its clock to
// stay within its power budget, so this rate sits below the published peak.
// The caller times the launch; the kernel writes one float per thread so that
// nothing is optimised away.  Not part of the attention path: it is built
// into its own library (libfa_probe.so, include/fa_probe.h).
#include <stdint.h>

#include "fa_device.h"
#include "fa_probe.h"

namespace fa {

namespace {
// splitmix-style 32-bit mixing of a counter: pseudo-random operand bits
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
// random bf16 in [1, 2) x sign (finite, normal)
__device__ __forceinline__ __bf16 rand_bf16(uint32_t seed) {
  const uint32_t r = mix32(seed);
  const uint16_t bits = (uint16_t)(0x3f80u | (r & 0x7fu) | ((r >> 8) & 0x8000u));
  return __builtin_bit_cast(__bf16, bits);
}
// random e4m3fn byte, never a NaN code (0x7f, 0xff)
__device__ __forceinline__ uint32_t rand_fp8x4(uint32_t seed) {
  uint32_t r = mix32(seed);
  uint32_t out = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t byte = (r >> (8 * b)) & 0xffu;
    if ((byte & 0x7fu) == 0x7fu) byte ^= 0x01u;
    out |= byte << (8 * b);
  }
  return out;
}
}  // namespace

template <bool FP8>
__global__ __launch_bounds__(512, 1) void mfma_peak_kernel(float* __restrict__ out, int iters) {
  const uint32_t seed = blockIdx.x * 512u + threadIdx.x;
  f32x16 c[4] = {};
  if constexpr (FP8) {
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (int)rand_fp8x4(seed * 16u + e);
      b[e] = (int)rand_fp8x4(seed * 16u + 8u + e);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int m = 0; m < 8; ++m) c[m & 3] = mfma_fp8_scaled<0, 0>(a, b, c[m & 3], 0x7f7f7f7fu, 0x7f7f7f7fu);
    }
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = rand_bf16(seed * 16u + e);
      b[e] = rand_bf16(seed * 16u + 8u + e);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int m = 0; m < 8; ++m) c[m & 3] = mfma_bf16(a, b, c[m & 3]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[k][i];
  out[blockIdx.x * 512u + threadIdx.x] = s;
}

}  // namespace fa

extern "C" int fa_measure_mfma_rate(float* out, int blocks, int iters, int dtype, void* stream) {
  if (dtype != FA_PROBE_BF16 && dtype != FA_PROBE_FP8_E4M3)
    return dtype == FA_PROBE_FP32 ? FA_PROBE_ERR_UNSUPPORTED : FA_PROBE_ERR_INVALID_ARG;
  if (!out || ((uintptr_t)out & 3u) != 0 || blocks < 1 || blocks > 65536 || iters < 1 ||
      iters > (1 << 20))
    return FA_PROBE_ERR_INVALID_ARG;
  const hipStream_t st = (hipStream_t)stream;
  if (dtype == FA_PROBE_FP8_E4M3)
    hipLaunchKernelGGL(fa::mfma_peak_kernel<true>, dim3(blocks), dim3(512), 0, st, out, iters);
  else
    hipLaunchKernelGGL(fa::mfma_peak_kernel<false>, dim3(blocks), dim3(512), 0, st, out, iters);
  return hipGetLastError() == hipSuccess ? FA_PROBE_OK : FA_PROBE_ERR_HIP;
}
