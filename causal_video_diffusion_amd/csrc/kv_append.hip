// RoPE the chunk's keys and append keys and values to the frame-slot ring
// (UnStep, abstract: the KV cache is indexed by latent frame, and RoPE is
// applied from precomputed coefficients).
//
// One workgroup handles 64 tokens of one latent frame for one head:
//   keys:   16-byte loads of k_new and of the table's cos/sin for four
//           rotation pairs, rotation in fp32, bf16 rounding, 16-byte stores
//           into the key slot [slot][h][t][:]  (a straight row copy);
//   values: 16-byte loads into an LDS tile [token][dim], then 16-byte stores
//           of 8 consecutive tokens per dimension into the transposed value
//           slot [slot][h][dim][t] (the layout the attention's PV product
//           reads without a transpose).
// With with_v == 0 only the keys are appended (the values reach the ring
// from the value projection's epilogue instead).
// The work is a streaming copy with no reuse (HBM-bound).  Workgroups are
// ordered head-fastest and XCD-aware, so the table rows of a token tile are
// fetched from HBM once and re-read by its other heads from the same L2.

#include "append_keys.h"
#include "ust_device.h"
#include "ust_internal.h"

namespace ust {
namespace {

constexpr int kTok = 64;  // tokens per workgroup

// map blockIdx to work so each XCD (8, dispatched round robin) gets a
// contiguous range: the heads of one token tile then share an L2 and the
// tile's table rows are fetched from HBM once
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int q = nb / 8, rem = nb % 8;
  const int x = b % 8, k = b / 8;
  return (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + k;
}

template <int D>
__global__ void __launch_bounds__(256)
kv_append_kernel(AppendArgs a) {
  constexpr int P = D / 2;
  constexpr int CH = D / 8;          // 16-byte chunks per head row
  constexpr int LROW = D / 2 + 1;    // LDS row stride in dwords (padded)
  constexpr int IT = (kTok * CH) / 256;
  __shared__ uint32_t vt[kTok * LROW];

  const int ntile = (a.T + kTok - 1) / kTok;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int h = w % a.H;                         // head fastest: one tile's heads are adjacent
  const int tile = w / a.H;
  const int fi = tile / ntile;                   // frame within the chunk
  const int t0 = (tile % ntile) * kTok;          // first token of the tile
  const int nt = min(kTok, a.T - t0);            // tokens here, a multiple of 8
  const int slot = a.chunk_slot[fi];
  const int64_t row0 = int64_t(fi) * a.T + t0;   // chunk token index of t0
  const int64_t tab0 = (int64_t(a.tab_frame) * a.T + row0) * P;
  const uint16_t* __restrict__ knew = a.k_new;
  const uint16_t* __restrict__ vnew = a.v_new;
  const float* __restrict__ ctab = a.cos_tab;
  const float* __restrict__ stab = a.sin_tab;

  // all loads first (nothing is stored before them, so they are in flight
  // together), then rotation and stores
  uint4 kw[IT], vw[IT];
  float4 cs[IT], sn[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = threadIdx.x + 256 * it;
    const int tl = min(c / CH, nt - 1);          // rows past the frame re-read the last one
    const int dc = c % CH;
    const int64_t src = ((row0 + tl) * a.H + h) * D + dc * 8;
    kw[it] = *reinterpret_cast<const uint4*>(knew + src);
    vw[it] = a.with_v ? *reinterpret_cast<const uint4*>(vnew + src) : make_uint4(0, 0, 0, 0);
    cs[it] = *reinterpret_cast<const float4*>(ctab + tab0 + int64_t(tl) * P + dc * 4);
    sn[it] = *reinterpret_cast<const float4*>(stab + tab0 + int64_t(tl) * P + dc * 4);
  }

  uint16_t* kdst = a.k_cache + ((int64_t(slot) * a.H + h) * a.T + t0) * D;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = threadIdx.x + 256 * it;
    const int tl = c / CH;
    const int dc = c % CH;
    if (tl < nt) {
      const uint32_t kin[4] = {kw[it].x, kw[it].y, kw[it].z, kw[it].w};
      const float c4[4] = {cs[it].x, cs[it].y, cs[it].z, cs[it].w};
      const float s4[4] = {sn[it].x, sn[it].y, sn[it].z, sn[it].w};
      uint32_t kout[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float r0, r1;
        rope_pair(bf16_lo(kin[e]), bf16_hi(kin[e]), c4[e], s4[e], r0, r1);
        kout[e] = pack_bf16x2(r0, r1);
      }
      *reinterpret_cast<uint4*>(kdst + int64_t(tl) * D + dc * 8) =
          make_uint4(kout[0], kout[1], kout[2], kout[3]);
      if (a.with_v) {
        uint32_t* row = vt + tl * LROW + dc * 4;
        row[0] = vw[it].x;
        row[1] = vw[it].y;
        row[2] = vw[it].z;
        row[3] = vw[it].w;
      }
    }
  }
  if (!a.with_v) return;   // uniform over the workgroup
  __syncthreads();

  // transposed values: item = (dim d, group of 8 tokens)
  uint16_t* vdst = a.v_cache + (int64_t(slot) * a.H + h) * D * a.TV + t0;
  const uint16_t* vt16 = reinterpret_cast<const uint16_t*>(vt);
#pragma unroll
  for (int it = 0; it < (D * (kTok / 8)) / 256; ++it) {
    const int c = threadIdx.x + 256 * it;
    const int tg = c % (kTok / 8);
    const int d = c / (kTok / 8);
    if (tg * 8 < nt) {
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = vt16[(tg * 8 + 2 * e) * (2 * LROW) + d];
        const uint32_t hi = vt16[(tg * 8 + 2 * e + 1) * (2 * LROW) + d];
        wv[e] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4*>(vdst + int64_t(d) * a.TV + tg * 8) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
  }
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s) {
  const int ntile = (a.T + kTok - 1) / kTok;
  dim3 grid(ntile * a.C * a.H);
  if (a.D == 128)
    hipLaunchKernelGGL(kv_append_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ust
