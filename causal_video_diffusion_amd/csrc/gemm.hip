// bf16 GEMM Y[M][N] = X[M][K] W[N][K]^T (+ bias), fp32 accumulation, bf16
// out: the two products of the truncated-SVD projections (UnStep, abstract:
// truncated SVD of the attention value and output projections), and the
// dense projection when the factor is a full weight.
//
// Design (gfx950, MFMA 32x32x16 bf16):
//  * The product is formed transposed, Y^T = W X^T, so each lane ends with
//    one output row m and runs of 4 consecutive columns n: 8-byte stores.
//  * Tiles BM x 128 (BM = 128 or 64) with BK = 64, 4 waves in a 2 x 2 grid,
//    both operand tiles k-contiguous in LDS with an XOR swizzle on 16-byte
//    chunks (conflict-free MFMA operand reads), double-buffered.
//  * Ragged M, N and K are zero-filled at the tile loads; stores are masked.

#include "ust_device.h"
#include "ust_internal.h"

namespace ust {
namespace {

constexpr int kBN = 128;
constexpr int kBK = 64;

template <int MB>  // 32-row blocks of X per wave; BM = 64 * MB
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_nt_kernel(GemmArgs g) {
  constexpr int BM = 64 * MB;
  constexpr int NB = 2;                  // 32-row blocks of W per wave
  constexpr int XITEMS = BM * 8 / 256;   // 16-byte chunks of the X tile per thread
  constexpr int WITEMS = kBN * 8 / 256;
  __shared__ __attribute__((aligned(16))) uint16_t lx[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t lw[2][kBN * kBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int wm = wave & 1;   // wave's position in the 2 x 2 grid
  const int wn = wave >> 1;
  const int nbn = (g.N + kBN - 1) / kBN;
  const int m0 = (blockIdx.x / nbn) * BM;
  const int n0 = (blockIdx.x % nbn) * kBN;
  const int nkt = (g.K + kBK - 1) / kBK;

  const int ch = tid & 7;    // chunk within a 64-wide k row
  const int r0 = tid >> 3;   // first row this thread loads; then +32 each item
  uint4 xr[XITEMS], wr[WITEMS];
  auto gload = [&](int kt) {
    const int k = kt * kBK + ch * 8;
#pragma unroll
    for (int it = 0; it < XITEMS; ++it) {
      const int m = m0 + r0 + 32 * it;
      xr[it] = make_uint4(0, 0, 0, 0);
      if (m < g.M && k < g.K) xr[it] = *reinterpret_cast<const uint4*>(g.x + int64_t(m) * g.K + k);
    }
#pragma unroll
    for (int it = 0; it < WITEMS; ++it) {
      const int n = n0 + r0 + 32 * it;
      wr[it] = make_uint4(0, 0, 0, 0);
      if (n < g.N && k < g.K) wr[it] = *reinterpret_cast<const uint4*>(g.w + int64_t(n) * g.K + k);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < XITEMS; ++it) {
      const int r = r0 + 32 * it;
      *reinterpret_cast<uint4*>(&lx[buf][r * kBK + ((ch ^ (r & 7)) * 8)]) = xr[it];
    }
#pragma unroll
    for (int it = 0; it < WITEMS; ++it) {
      const int r = r0 + 32 * it;
      *reinterpret_cast<uint4*>(&lw[buf][r * kBK + ((ch ^ (r & 7)) * 8)]) = wr[it];
    }
  };

  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  gload(0);
  lstore(0);
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    __syncthreads();
    const bool more = kt + 1 < nkt;
    if (more) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int c = 2 * s + half;
      bf16x8 wf[NB], xf[MB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int r = wn * 32 * NB + 32 * i + l32;
        wf[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&lw[buf][r * kBK + ((c ^ (r & 7)) * 8)]));
      }
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int r = wm * 32 * MB + 32 * j + l32;
        xf[j] = as_bf16x8(*reinterpret_cast<const uint4*>(&lx[buf][r * kBK + ((c ^ (r & 7)) * 8)]));
      }
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) acc[i][j] = mfma32(wf[i], xf[j], acc[i][j]);
    }
    if (more) lstore(buf ^ 1);
  }

  // epilogue: lane holds row m = ... + l32 and columns n = 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int m = m0 + wm * 32 * MB + 32 * j + l32;
    if (m >= g.M) continue;
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 32 * NB + 32 * i + 8 * q + 4 * half;
        if (n >= g.N) continue;   // N % 8 == 0, so n..n+3 are all in or all out
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[i][j][4 * q + e];
          if (g.bias) v[e] += bf16_lo(g.bias[n + e]);
        }
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(g.y + int64_t(m) * g.N + n) = o;
      }
  }
}

}  // namespace

hipError_t launch_gemm_nt(const GemmArgs& g, hipStream_t s) {
  const int nbn = (g.N + kBN - 1) / kBN;
  const int tiles128 = ((g.M + 127) / 128) * nbn;
  // enough workgroups to cover the 256 CUs twice, else halve the row tile
  if (tiles128 >= 512) {
    dim3 grid(tiles128);
    hipLaunchKernelGGL(gemm_nt_kernel<2>, grid, dim3(256), 0, s, g);
  } else {
    dim3 grid(((g.M + 63) / 64) * nbn);
    hipLaunchKernelGGL(gemm_nt_kernel<1>, grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace ust
