// One step of the chunk sampler (UnStep, Table 4: the shift-5 noise levels
// and the clean-cache level; abstract: the generated frames are renoised to a
// nearly clean level and refined by the clean-cache forward).  Under the
// flow-matching parameterisation of this model family a latent at level
// sigma is (1 - sigma) x0 + sigma eps and the DiT returns the velocity
// eps - x0, so a step is elementwise:
//   x0_hat = x - sigma v                     (one fused multiply-add)
//   x_next = (1 - sigma') x0_hat + sigma' eps'   ((1 - sigma') x0_hat rounded,
//                                                 then one fused multiply-add)
// Streaming and HBM-bound: each thread takes 4 elements (16-byte fp32 loads
// and stores, 8-byte bf16 velocity loads), grid-stride; the 0-3 trailing
// elements are done one per thread.  Every output element depends only on
// the inputs at its own index, so the outputs may be the inputs' buffers.

#include "ust_device.h"
#include "ust_internal.h"

namespace ust {
namespace {

__device__ __forceinline__ void step1(float x, float v, float e, const FlowStepArgs& a, float& x0,
                                      float& xn) {
  x0 = fmaf(-a.sigma, v, x);
  xn = a.noise ? fmaf(a.sigma_next, e, a.keep * x0) : x0;
}

__global__ void __launch_bounds__(256) flow_step_kernel(FlowStepArgs a) {
  const int64_t n4 = a.n / 4;
  const int64_t first = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = first; i < n4; i += stride) {
    const float4 x = reinterpret_cast<const float4*>(a.x)[i];
    const uint2 vw = reinterpret_cast<const uint2*>(a.v)[i];
    float4 e = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.noise) e = reinterpret_cast<const float4*>(a.noise)[i];
    float4 x0, xn;
    step1(x.x, bf16_lo(vw.x), e.x, a, x0.x, xn.x);
    step1(x.y, bf16_hi(vw.x), e.y, a, x0.y, xn.y);
    step1(x.z, bf16_lo(vw.y), e.z, a, x0.z, xn.z);
    step1(x.w, bf16_hi(vw.y), e.w, a, x0.w, xn.w);
    if (a.x0_out) reinterpret_cast<float4*>(a.x0_out)[i] = x0;
    reinterpret_cast<float4*>(a.x_next)[i] = xn;
  }
  const int64_t t = 4 * n4 + first;   // trailing elements
  if (first < a.n - 4 * n4) {
    const uint16_t vh = a.v[t];
    float x0, xn;
    step1(a.x[t], __uint_as_float(uint32_t(vh) << 16), a.noise ? a.noise[t] : 0.f, a, x0, xn);
    if (a.x0_out) a.x0_out[t] = x0;
    a.x_next[t] = xn;
  }
}

}  // namespace

hipError_t launch_flow_step(const FlowStepArgs& a, hipStream_t s) {
  const int64_t n4 = a.n / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(flow_step_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ust
