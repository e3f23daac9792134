// Measurement aid, not a step of the path: a kernel that only issues bf16
// MFMAs, so that a benchmark can state the rate this part actually sustains
// beside the published peak.  The sustained rate depends on the operands:
// the shader clock under a matrix load is power-limited, and operands whose
// bits toggle (as real activations and weights do) draw more power than
// constant or zero ones, so the operands here are pseudo-random bf16 values
// of magnitude 0.5 .. 2 with random signs and mantissas.
//
// Every wave keeps four independent 32x32x16 accumulators and four operand
// pairs, and issues one MFMA per accumulator per round for `iters` rounds,
// cycling through the operand pairs: no memory traffic, no VALU work in the
// loop.  Two waves per SIMD (8 per workgroup) keep the matrix pipe fed.
// Each wave writes one sum of its accumulators, so the work is not removed.

#include "ust_device.h"
#include "ust_internal.h"

namespace ust {
namespace {

constexpr int kCalibAcc = 4;

// 32-bit integer hash (the "lowbias32" xor-shift-multiply mixer)
__device__ __forceinline__ uint32_t calib_hash(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du;
  x ^= x >> 15; x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// bf16 with a random sign, exponent 126 or 127 and a random mantissa
__device__ __forceinline__ __bf16 calib_operand(uint32_t key) {
  const uint32_t h = calib_hash(key);
  const uint16_t bits = uint16_t((h & 0x8000u) | 0x3f00u | ((h >> 16) & 0xffu));
  return __builtin_bit_cast(__bf16, bits);
}

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
calib_mfma_kernel(int32_t iters, float* out) {
  const uint32_t gid = blockIdx.x * 512u + threadIdx.x;
  bf16x8 a[kCalibAcc], b[kCalibAcc];
#pragma unroll
  for (int o = 0; o < kCalibAcc; ++o)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[o][i] = calib_operand(gid * 64u + o * 16u + i);
      b[o][i] = calib_operand(gid * 64u + o * 16u + 8u + i);
    }
  f32x16 acc[kCalibAcc];
#pragma unroll
  for (int j = 0; j < kCalibAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  int32_t it = 0;
  for (; it + 4 <= iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < kCalibAcc; ++j)
        acc[j] = mfma32(a[(u + j) & 3], b[(u + 2 * j) & 3], acc[j]);
  }
  for (; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kCalibAcc; ++j) acc[j] = mfma32(a[j], b[j], acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kCalibAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 8 + (threadIdx.x >> 6)] = s;
}

}  // namespace

double calib_mfma_flops(int32_t n_wg, int32_t iters) {
  return double(n_wg) * 8.0 * double(iters) * kCalibAcc * (2.0 * 32 * 32 * 16);
}

hipError_t launch_calib_mfma(int32_t n_wg, int32_t iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(calib_mfma_kernel, dim3(n_wg), dim3(512), 0, s, iters, out);
  return hipGetLastError();
}

}  // namespace ust
