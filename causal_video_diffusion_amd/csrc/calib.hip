// Measurement aid, not a step of the path: a kernel that only issues bf16
// MFMAs, so that a benchmark can state the rate this part actually sustains
// (its shader clock under a sustained matrix load sits below the nominal
// 2.4 GHz) beside the published peak.
//
// Every wave keeps four independent 32x32x16 accumulators and issues their
// MFMAs back to back for `iters` rounds: no memory traffic, no VALU work in
// the loop.  Two waves per SIMD (8 per workgroup) keep the matrix pipe fed.
// Each wave writes one sum of its accumulators, so the work is not removed.

#include "ust_device.h"
#include "ust_internal.h"

namespace ust {
namespace {

constexpr int kCalibAcc = 4;

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
calib_mfma_kernel(int32_t iters, float* out) {
  const int lane = threadIdx.x & 63;
  // small exact operands (2^-8 and +-2^-9) keep every sum finite
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0x1p-8f);
    b[i] = (__bf16)(((lane + i) & 1) ? 0x1p-9f : -0x1p-9f);
  }
  f32x16 acc[kCalibAcc];
#pragma unroll
  for (int j = 0; j < kCalibAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kCalibAcc; ++j) acc[j] = mfma32(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kCalibAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (lane == 0) out[blockIdx.x * 8 + (threadIdx.x >> 6)] = s;
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
