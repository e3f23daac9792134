// Causal 3-D convolution of the decoder stack (UnStep, abstract: the VAE
// decoder runs with an optimised memory layout, precision and convolution
// kernels; Table 3: the decoder turns 21 latent frames of 16 x 60 x 104 into
// 81 frames of 832 x 480).  Output frame t reads input frames t-2 .. t (zero
// before the first), rows and columns with zero padding 1, stride 1.
//
// Layout and precision: activations channels last [T][H][W][C] bf16, weights
// [Cout][3][3][3][Cin] bf16, bias fp32, fp32 accumulation, bf16 out.  With
// the channels innermost, 8 consecutive input channels of one position are
// one 16-byte load, which is exactly a lane's share of an MFMA operand.
//
// Implicit GEMM on bf16 MFMA 32x32x16: out^T[co][p] = sum over taps and
// 16-channel steps of W[co][tap][ci] x[p shifted by the tap][ci].
//  * A operand, the weights: one tap's [128 co][Cin] block per step, staged
//    global -> registers -> LDS (two buffers, 16-byte chunks XOR-swizzled by
//    row so each MFMA operand read hits distinct banks) and shared by the
//    workgroup's 8 waves.
//  * B operand, the input: each lane loads its own position's 8 channels at
//    the tap's offset straight into registers (zero outside the input),
//    four k-steps ahead of the MFMA that uses them.
//  * A workgroup owns 256 consecutive positions of the flattened (t, y, x)
//    grid (32 per wave) and 128 output channels; workgroups are ordered so
//    that each XCD takes a contiguous run of positions.
//  * Each lane ends with 4 consecutive output channels of one position per
//    register group: 8-byte stores.

#include "ust_device.h"
#include "ust_internal.h"

namespace ust {
namespace {

constexpr int kConvWaves = 8;
constexpr int kConvCo = 128;   // output channels per workgroup
constexpr int kConvPf = 4;     // input fragments in flight per wave

__device__ __forceinline__ int conv_xcd_remap(int b, int nb) {
  const int q = nb / 8, rem = nb % 8;
  const int x = b % 8, k = b / 8;
  return (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + k;
}

// XOR key of weight row `row` for rows of nch 16-byte chunks (a power of
// two): the 16 rows one 16-lane group reads land on 16 distinct bank groups
__device__ __forceinline__ int conv_key(int row, int nch) {
  return nch >= 16 ? (row & 15) : ((row / (16 / nch)) & (nch - 1));
}

template <int Ci>
__global__ void __launch_bounds__(64 * kConvWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
conv3d_causal_kernel(ConvArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t wl[2 * kConvCo * Ci];   // two taps' weights
  const int Co = a.Co;
  constexpr int nch = Ci / 8;             // 16-byte chunks per weight row
  constexpr int nks = Ci / 16;            // k-steps per tap
  constexpr int total = 27 * nks;         // k-steps in all
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int HW = a.H * a.W;
  const int64_t P = int64_t(a.T) * HW;
  const int ntile = int((P + 255) / 256);
  const int tile = conv_xcd_remap(blockIdx.x, ntile);
  const int co0 = blockIdx.y * kConvCo;

  // this lane's position and the taps that stay inside the input
  const int64_t p = int64_t(tile) * 256 + wave * 32 + l32;
  const bool pvalid = p < P;
  const int pp = pvalid ? int(p) : 0;
  const int pt = pp / HW, pr = pp - pt * HW, py = pr / a.W, px = pr - py * a.W;
  uint32_t tapmask = 0;
#pragma unroll
  for (int tap = 0; tap < 27; ++tap) {
    const int dt = tap / 9, dy = (tap / 3) % 3, dx = tap % 3;
    const int t2 = pt + dt - 2, y2 = py + dy - 1, x2 = px + dx - 1;
    if (pvalid && t2 >= 0 && y2 >= 0 && y2 < a.H && x2 >= 0 && x2 < a.W) tapmask |= 1u << tap;
  }
  const uint16_t* xbase = a.x + int64_t(pp) * Ci + 8 * half;

  // input fragment of flattened k-step s (tap s / nks, channels 16 (s % nks) ..)
  auto load_in = [&](int s) __attribute__((always_inline)) -> uint4 {
    const int tap = s / nks, c = s - tap * nks;
    const int dt = tap / 9, dy = (tap / 3) % 3, dx = tap % 3;
    const int64_t delta = (int64_t(dt - 2) * HW + (dy - 1) * a.W + (dx - 1)) * Ci + 16 * c;
    const bool ok = (tapmask >> tap) & 1u;
    const uint4 v = *reinterpret_cast<const uint4*>(xbase + (ok ? delta : int64_t(16 * c)));
    return ok ? v : make_uint4(0, 0, 0, 0);
  };

  // weights of one tap: chunk q of the [128][Ci] block
  constexpr int wchunks = kConvCo * nch;
  constexpr int wper = (wchunks + 64 * kConvWaves - 1) / (64 * kConvWaves);
  uint4 wreg[wper];
  auto load_w = [&](int tap) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < wper; ++i) {
      const int q = tid + i * 64 * kConvWaves;
      if (q < wchunks) {
        const int row = q / nch, c = q - row * nch;
        wreg[i] = *reinterpret_cast<const uint4*>(a.w + (int64_t(co0 + row) * 27 + tap) * Ci + c * 8);
      }
    }
  };
  auto store_w = [&](int buf) __attribute__((always_inline)) {
    uint16_t* dst = wl + buf * kConvCo * Ci;
#pragma unroll
    for (int i = 0; i < wper; ++i) {
      const int q = tid + i * 64 * kConvWaves;
      if (q < wchunks) {
        const int row = q / nch, c = q - row * nch;
        *reinterpret_cast<uint4*>(dst + row * Ci + ((c ^ conv_key(row, nch)) * 8)) = wreg[i];
      }
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;

  uint4 inq[kConvPf];
#pragma unroll
  for (int i = 0; i < kConvPf; ++i) inq[i] = i < total ? load_in(i) : make_uint4(0, 0, 0, 0);
  load_w(0);
  store_w(0);
  __syncthreads();

  int s = 0;
  for (int tap = 0; tap < 27; ++tap) {
    const int buf = tap & 1;
    if (tap + 1 < 27) load_w(tap + 1);   // lands in registers while this tap computes
    const uint16_t* W = wl + buf * kConvCo * Ci;
#pragma unroll
    for (int c = 0; c < nks; ++c, ++s) {
      const bf16x8 bf = as_bf16x8(inq[0]);
#pragma unroll
      for (int i = 0; i + 1 < kConvPf; ++i) inq[i] = inq[i + 1];
      inq[kConvPf - 1] = s + kConvPf < total ? load_in(s + kConvPf) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int row = 32 * b + l32;
        const bf16x8 af = as_bf16x8(
            *reinterpret_cast<const uint4*>(W + row * Ci + (((2 * c + half) ^ conv_key(row, nch)) * 8)));
        acc[b] = mfma32(af, bf, acc[b]);
      }
    }
    if (tap + 1 < 27) store_w(buf ^ 1);   // the other buffer was last read a tap ago
    __syncthreads();
  }

  // lane: position p, output channels co0 + 32 b + 8 (r / 4) + 4 half + r % 4
  if (pvalid) {
    uint16_t* yp = a.y + p * Co + co0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int co = 32 * b + 8 * g + 4 * half;
        float v[4] = {acc[b][4 * g], acc[b][4 * g + 1], acc[b][4 * g + 2], acc[b][4 * g + 3]};
        if (a.bias) {
          const float4 bb = *reinterpret_cast<const float4*>(a.bias + co0 + co);
          v[0] += bb.x; v[1] += bb.y; v[2] += bb.z; v[3] += bb.w;
        }
        *reinterpret_cast<uint2*>(yp + co) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
  }
}

}  // namespace

hipError_t launch_conv3d_causal(const ConvArgs& a, hipStream_t s) {
  const int64_t P = int64_t(a.T) * a.H * a.W;
  const dim3 grid(unsigned((P + 255) / 256), unsigned(a.Co / kConvCo));
  const dim3 block(64 * kConvWaves);
  switch (a.Ci) {
    case 16: hipLaunchKernelGGL(conv3d_causal_kernel<16>, grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL(conv3d_causal_kernel<32>, grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL(conv3d_causal_kernel<64>, grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(conv3d_causal_kernel<128>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ust
