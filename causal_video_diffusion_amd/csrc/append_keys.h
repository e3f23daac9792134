// The keys' half of the KV append (UnStep, abstract: RoPE applied from
// precomputed coefficients, the KV cache indexed by latent frame) as a
// device function that a group of threads runs inside a larger kernel: the
// first product of the value projection runs it in workgroups beyond its
// own tiles, on compute units the product leaves idle.
//
// A key tile is 64 tokens of one latent frame for one head, numbered head
// fastest, as in kv_append_kernel, with the same arithmetic: 16-byte loads
// of k_new and of the table's cos/sin for four rotation pairs, the rotation
// in fp32, one bf16 rounding, 16-byte stores into [slot][h][t][:].
#pragma once

#include "ust_device.h"
#include "ust_internal.h"

namespace ust {

// RoPE of one pair (x0, x1) by the angle whose cosine and sine are c and s,
// in fp32 with the fused multiply-adds written out, so that every kernel
// that rotates a key from the cached table rounds the same way:
//   r0 = x0 c - x1 s  as fma(x0, c, -(x1 s))
//   r1 = x0 s + x1 c  as fma(x1, c, x0 s)
__device__ __forceinline__ void rope_pair(float x0, float x1, float c, float s, float& r0,
                                          float& r1) {
  r0 = __builtin_fmaf(x0, c, -(x1 * s));
  r1 = __builtin_fmaf(x1, c, x0 * s);
}

constexpr int kKeyTileTok = 64;   // tokens per key tile

// key tiles of a chunk of C frames of T tokens and H heads
__host__ __device__ inline int key_tiles(int T, int C, int H) {
  return ((T + kKeyTileTok - 1) / kKeyTileTok) * C * H;
}

// Key tile w (0 <= w < key_tiles) by NTH threads; i is this thread's index
// among them.  All loads are issued before any store.
template <int D, int NTH>
__device__ __forceinline__ void append_key_tile(const AppendArgs& a, int w, int i) {
  constexpr int P = D / 2;
  constexpr int CH = D / 8;                        // 16-byte chunks per head row
  constexpr int IT = (kKeyTileTok * CH) / NTH;     // chunks per thread
  static_assert(IT * NTH == kKeyTileTok * CH, "a tile's chunks split evenly over the threads");
  const int ntile = (a.T + kKeyTileTok - 1) / kKeyTileTok;
  const int h = w % a.H;
  const int tile = w / a.H;
  const int fi = tile / ntile;                     // frame within the chunk
  const int t0 = (tile % ntile) * kKeyTileTok;     // first token of the tile
  const int nt = min(kKeyTileTok, a.T - t0);       // tokens here, a multiple of 8
  const int64_t row0 = int64_t(fi) * a.T + t0;     // chunk token index of t0
  const int64_t tab0 = (int64_t(a.tab_frame) * a.T + row0) * P;
  uint4 kw[IT];
  float4 cs[IT], sn[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = i + NTH * it;
    const int tl = min(c / CH, nt - 1);            // rows past the frame re-read the last one
    const int dc = c % CH;
    kw[it] = *reinterpret_cast<const uint4*>(a.k_new + ((row0 + tl) * a.H + h) * D + dc * 8);
    cs[it] = *reinterpret_cast<const float4*>(a.cos_tab + tab0 + int64_t(tl) * P + dc * 4);
    sn[it] = *reinterpret_cast<const float4*>(a.sin_tab + tab0 + int64_t(tl) * P + dc * 4);
  }
  uint16_t* kdst = a.k_cache + ((int64_t(a.chunk_slot[fi]) * a.H + h) * a.T + t0) * D;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = i + NTH * it;
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
    }
  }
}

}  // namespace ust
