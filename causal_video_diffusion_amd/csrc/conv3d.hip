// Causal 3-D convolution of the decoder stack (UnStep, abstract: the VAE
// decoder runs with an optimised memory layout, precision and convolution
// kernels; Table 3: the decoder turns 21 latent frames of 16 x 60 x 104 into
// 81 frames of 832 x 480).  Output frame t reads input frames t-2 .. t (zero
// before the first; in the streaming form, for a clip decoded chunk by
// chunk, x starts with two history frames that take the padding's place),
// rows and columns with zero padding 1, stride 1.
//
// Layout and precision: activations channels last [T][H][W][C] bf16, weights
// [Cout][3][3][3][Cin] bf16, bias fp32, fp32 accumulation, bf16 out.  With
// the channels innermost, the input rows a tap needs are one contiguous
// block of memory for a run of consecutive positions.
//
// Implicit GEMM on bf16 MFMA 32x32x16: out^T[co][p] = sum over taps and
// channels of W[co][tap][ci] x[p shifted by the tap][ci].
//  * A workgroup owns 512 consecutive positions of the flattened (t, y, x)
//    grid (64 per wave, two 32-position blocks) and 128 output channels
//    (four 32-channel blocks): 8 MFMAs per 16 channels, each input fragment
//    used 4 times and each weight fragment twice.
//  * Work runs in stages of one (frame offset dt, row offset dy) and CQ
//    input channels: the 514 input positions the three column offsets dx
//    need (one contiguous block, clamped to the tensor) and the three taps'
//    weights go global -> LDS (global_load_lds, coalesced 64-byte rows,
//    16-byte chunks XOR-swizzled so operand reads hit distinct banks),
//    double-buffered: stage s+1 loads while stage s computes.
//  * Within a stage the operand fragments of the next (tap, 16 channels)
//    step are read from LDS between the current step's MFMAs, so the matrix
//    pipe does not wait on LDS latency at each step.
//  * Taps that leave the input (frames before the first, rows off the
//    frame, columns that would wrap into the next row) are zeroed per
//    position after the fragment read.
//  * Each lane ends with 4 consecutive output channels of one position per
//    register group: 8-byte stores.  Co is a multiple of 32: in a last,
//    partly empty 128-channel tile the missing weight rows load a clamped
//    (finite) row and their outputs are not stored.

#include <type_traits>

#include "ust_device.h"
#include "ust_internal.h"

namespace ust {
namespace {

constexpr int kConvWaves = 8;
constexpr int kConvCo = 128;               // output channels per workgroup
constexpr int kConvPos = 64 * kConvWaves;  // positions per workgroup
constexpr int kConvRows = kConvPos + 32;   // staged input rows (514 used; whole 1 KB loads)

__device__ __forceinline__ int conv_xcd_remap(int b, int nb) {
  const int q = nb / 8, rem = nb % 8;
  const int x = b % 8, k = b / 8;
  return (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + k;
}

__device__ __forceinline__ uint32_t conv_lds_addr(const uint16_t* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint16_t*)(p)));
}
// 16 bytes per lane, global -> LDS at m0 + 16 * lane.  The base is made
// wave-uniform through readfirstlane; the asm starts with s_nop 4 because a
// vector instruction's write of a scalar register is not interlocked with a
// vector memory read of it (5 wait states) and the compiler adds none
// before inline asm.
__device__ __forceinline__ void conv_load_lds16(const uint16_t* sbase, uint32_t voff_bytes, uint32_t m0) {
  const uint64_t p = reinterpret_cast<uint64_t>(sbase);
  const uint64_t su = (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(p >> 32)))) << 32) |
                      uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(p))));
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff_bytes),
               "s"(reinterpret_cast<const uint16_t*>(su)), "{m0}"(m0));
}
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ void conv_wait_all() {
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (0 << 8) | (0 << 14));   // vmcnt(0) lgkmcnt(0)
}
__device__ __forceinline__ void conv_barrier() { asm volatile("s_barrier" ::: "memory"); }

// XOR key of a staged row of NCH 16-byte chunks (2 or 4): the 16
// consecutive rows one 16-lane group reads land on 16 distinct bank groups
template <int NCH>
__device__ __forceinline__ int conv_key(int row) {
  if constexpr (NCH == 4) return (row >> 2) & 3;
  else return (row >> 3) & 1;
}

// CQ input channels per stage: 16 when Ci is 16, else 32 (Ci a multiple of
// 32).  CI is Ci as a compile-time constant for the common widths (its index
// arithmetic then folds), or 0 to take Ci from the arguments.
template <int CQ, int CI>
__global__ void __launch_bounds__(64 * kConvWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
conv3d_causal_kernel(ConvArgs a) {
  constexpr int NCH = CQ / 8;                 // 16-byte chunks per staged row
  const int Ci = CI ? CI : a.Ci;
  const int NQ = Ci / CQ;                     // channel groups
  const int NSTAGE = 9 * NQ;                  // (dt, dy, channel group)
  constexpr int KS = CQ / 16;                 // k-steps per tap per stage
  constexpr int IN_EL = kConvRows * CQ;       // input block elements
  constexpr int W_EL = 3 * kConvCo * CQ;      // three taps' weights
  constexpr int BUF = IN_EL + W_EL;
  constexpr int IN_LOADS = IN_EL * 2 / 1024;  // 1 KB loads per stage
  constexpr int W_LOADS = W_EL * 2 / 1024;
  constexpr int NLOADS = IN_LOADS + W_LOADS;
  constexpr int LPW = (NLOADS + kConvWaves - 1) / kConvWaves;
  static_assert(IN_EL * 2 % 1024 == 0 && W_EL * 2 % 1024 == 0, "whole 1 KB loads");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * BUF];

  const int Co = a.Co;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int HW = a.H * a.W;
  const int P = a.T * HW;
  const int ntile = (P + kConvPos - 1) / kConvPos;
  const int tile = conv_xcd_remap(blockIdx.x, ntile);
  const int co0 = blockIdx.y * kConvCo;
  const int p0 = tile * kConvPos;

  // frames before frame 0: zero padding, or the two history frames at the
  // start of x (then input position p lives at x[p + 2 H W])
  const int t_lo = a.hist ? -2 : 0;
  const int pos_lo = t_lo * HW;
  // the taps each of this lane's two positions may read
  uint32_t tapmask[2];
#pragma unroll
  for (int pb = 0; pb < 2; ++pb) {
    const int p = p0 + wave * 64 + pb * 32 + l32;
    uint32_t m = 0;
    if (p < P) {
      const int pt = p / HW, pr = p - pt * HW, py = pr / a.W, px = pr - py * a.W;
#pragma unroll
      for (int tap = 0; tap < 27; ++tap) {
        const int t2 = pt + tap / 9 - 2, y2 = py + (tap / 3) % 3 - 1, x2 = px + tap % 3 - 1;
        if (t2 >= t_lo && y2 >= 0 && y2 < a.H && x2 >= 0 && x2 < a.W) m |= 1u << tap;
      }
    }
    tapmask[pb] = m;
  }

  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(conv_lds_addr(lds));
  // stage s: (dt, dy) = (s / NQ) / 3, % 3; channels CQ * (s % NQ) ..
  // loads I0 .. I1-1 (of LPW) of this wave's share of stage s into buffer buf
  auto issue = [&](int s, int buf, auto i0c, auto i1c) __attribute__((always_inline)) {
    constexpr int I0 = decltype(i0c)::value, I1 = decltype(i1c)::value;
    const int dtdy = s / NQ, q = s - dtdy * NQ;
    const int dt = dtdy / 3, dy = dtdy - 3 * dt;
    const int shift = (dt - 2) * HW + (dy - 1) * a.W - 1;   // input position of local row 0
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      const int li = wave * LPW + i;                        // 1 KB load index
      if (li < NLOADS) {
        const int e = li * 512 + lane * 8;                  // element of this lane's chunk
        const uint32_t dst = lds_base + uint32_t(buf * BUF + li * 512) * 2u;
        if (li < IN_LOADS) {
          const int row = e / CQ, cp = (e % CQ) / 8;
          const int c = cp ^ conv_key<NCH>(row);
          int pos = p0 + shift + row;
          pos = pos < pos_lo ? pos_lo : (pos >= P ? P - 1 : pos);  // clamped; such taps are masked
          conv_load_lds16(a.x, uint32_t(((pos - pos_lo) * Ci + q * CQ + c * 8) * 2), dst);
        } else {
          const int ew = e - IN_EL;
          const int row = ew / CQ, cp = (ew % CQ) / 8;       // row = dx * 128 + co
          const int c = cp ^ conv_key<NCH>(row);
          const int dx = row / kConvCo, co = min(co0 + row - dx * kConvCo, a.Co - 1);
          const int tap = dt * 9 + dy * 3 + dx;     // (rows past Co: clamped, never stored)
          conv_load_lds16(a.w, uint32_t(((co * 27 + tap) * Ci + q * CQ + c * 8) * 2), dst);
        }
      }
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int pb = 0; pb < 2; ++pb)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[pb][b][r] = 0.f;

  // stage s from buffer buf; between its 3 KS steps of 8 MFMAs, this
  // wave's loads of stage s + 1 (if any) go out a share at a time, so the
  // waves of a SIMD do not all stall on load issue at once
  constexpr int NSTEP = 3 * KS;
  auto compute = [&](int s, int buf, bool next) __attribute__((always_inline)) {
    const int dtdy = s / NQ;
    const uint16_t* X = lds + buf * BUF;
    const uint16_t* Wt = X + IN_EL;
    // fragments of two steps: step j's feed its MFMAs while step j+1's are read
    bf16x8 bfr[2][2], afr[2][4];
    auto rd = [&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      constexpr int dx = j / KS, k = j % KS, PAR = j & 1;
      const int tap = dtdy * 3 + dx;
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        const int row = wave * 64 + pb * 32 + l32 + dx;
        uint4 v = *reinterpret_cast<const uint4*>(X + row * CQ + (((2 * k + half) ^ conv_key<NCH>(row)) * 8));
        if (!((tapmask[pb] >> tap) & 1u)) v = make_uint4(0, 0, 0, 0);
        bfr[PAR][pb] = as_bf16x8(v);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int row = dx * kConvCo + 32 * b + l32;
        afr[PAR][b] = as_bf16x8(*reinterpret_cast<const uint4*>(Wt + row * CQ + (((2 * k + half) ^ conv_key<NCH>(row)) * 8)));
      }
    };
    rd(std::integral_constant<int, 0>{});
    static_for<0, NSTEP>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int PAR = j & 1;
      if (next)
        issue(s + 1, buf ^ 1, std::integral_constant<int, j * LPW / NSTEP>{},
              std::integral_constant<int, (j + 1) * LPW / NSTEP>{});
      if constexpr (j + 1 < NSTEP) rd(std::integral_constant<int, j + 1>{});
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) acc[pb][b] = mfma32(afr[PAR][b], bfr[PAR][pb], acc[pb][b]);
      if constexpr (j + 1 < NSTEP) {
        // one MFMA, then the next step's six reads one per MFMA, then the rest
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        static_for<0, 6>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        });
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    });
  };

  issue(0, 0, std::integral_constant<int, 0>{}, std::integral_constant<int, LPW>{});
  for (int s = 0; s < NSTAGE; ++s) {
    conv_wait_all();     // this wave's loads of stage s have landed
    conv_barrier();      // everyone's have, and stage s-1's buffer is free
    compute(s, s & 1, s + 1 < NSTAGE);
  }

  // lane: positions p0 + wave*64 + pb*32 + l32, output channels
  // co0 + 32 b + 8 (r / 4) + 4 half + r % 4
#pragma unroll
  for (int pb = 0; pb < 2; ++pb) {
    const int p = p0 + wave * 64 + pb * 32 + l32;
    if (p >= P) continue;
    uint16_t* yp = a.y + int64_t(p) * Co + co0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (co0 + 32 * b >= Co) break;   // Co is a multiple of 32
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int co = 32 * b + 8 * g + 4 * half;
        float v[4] = {acc[pb][b][4 * g], acc[pb][b][4 * g + 1], acc[pb][b][4 * g + 2], acc[pb][b][4 * g + 3]};
        if (a.bias) {
          const float4 bb = *reinterpret_cast<const float4*>(a.bias + co0 + co);
          v[0] += bb.x; v[1] += bb.y; v[2] += bb.z; v[3] += bb.w;
        }
        *reinterpret_cast<uint2*>(yp + co) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }
}

}  // namespace

hipError_t launch_conv3d_causal(const ConvArgs& a, hipStream_t s) {
  const int64_t P = int64_t(a.T) * a.H * a.W;
  const dim3 grid(unsigned((P + kConvPos - 1) / kConvPos), unsigned((a.Co + kConvCo - 1) / kConvCo));
  const dim3 block(64 * kConvWaves);
  if (a.Co % 32 != 0) return hipErrorInvalidValue;
  switch (a.Ci) {
    case 16: hipLaunchKernelGGL((conv3d_causal_kernel<16, 16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((conv3d_causal_kernel<32, 32>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((conv3d_causal_kernel<32, 64>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((conv3d_causal_kernel<32, 128>), grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL((conv3d_causal_kernel<32, 256>), grid, block, 0, s, a); break;
    case 512: hipLaunchKernelGGL((conv3d_causal_kernel<32, 512>), grid, block, 0, s, a); break;
    default:
      if (a.Ci <= 0 || a.Ci % 32 != 0) return hipErrorInvalidValue;
      hipLaunchKernelGGL((conv3d_causal_kernel<32, 0>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ust
