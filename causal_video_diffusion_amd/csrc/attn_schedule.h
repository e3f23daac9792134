// Integer schedule of the key-split attention: which (head, query tile, key
// tiles) each workgroup computes, and where a split unit's partial results
// go.  Host and device share this code; it touches no memory.
//
// A unit is one (head, 256-query tile).  Its work is its key tiles
// 0 .. ntiles-1.  Units in order, each unit's key tiles in order, form one
// sequence of total = n_units * ntiles steps, cut into G contiguous ranges:
// workgroup b owns steps [start(b), start(b + 1)), start(b) = b * total / G.
// A range meets one or more units; its part of each unit is a segment.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace ust {

// n / d for n >= 0, d > 0, in 32-bit arithmetic when both fit (a 64-bit
// division is a long instruction sequence on the GPU)
__host__ __device__ inline int64_t div_nonneg(int64_t n, int64_t d) {
  if (n < (int64_t(1) << 32) && d < (int64_t(1) << 32)) return int64_t(uint32_t(n) / uint32_t(d));
  return n / d;
}

// workgroups actually launched for `requested`: at most one per step
__host__ __device__ inline int attn_grid(int64_t total, int requested) {
  return int(total < requested ? total : requested);
}

__host__ __device__ inline int64_t wg_range_start(int b, int64_t total, int G) {
  return div_nonneg(int64_t(b) * total, G);
}

// the workgroup whose range holds step x: the largest b with start(b) <= x
__host__ __device__ inline int wg_of_step(int64_t x, int64_t total, int G) {
  int b = int(div_nonneg(x * G, total));
  while (b + 1 < G && wg_range_start(b + 1, total, G) <= x) ++b;
  return b;
}

struct AttnSegment {
  int unit;      // (head, query tile) index
  int k0;        // first key tile
  int n;         // key tiles, k0 .. k0 + n - 1
  int slot;      // -1: the whole unit (final output), else the partial slot
  int64_t next;  // first step after this segment
};

// The segment of workgroup w (range [xb, xe)) that starts at step x.
// Key order: when a unit is split, the workgroup holding its first step
// reaches it late in its own range; it takes the unit's last key tiles, and
// the later workgroups take key tiles from 0 upward.  So at any moment the
// workgroups on one head read keys near the same position, and no segment
// wraps around the unit's key sequence.
// Partial slots: 2w for the range's first segment, 2w + 1 for its last.
__host__ __device__ inline AttnSegment attn_segment(int64_t x, int64_t xb, int64_t xe, int w,
                                                    int ntiles, int64_t total, int G) {
  AttnSegment s;
  s.unit = int(div_nonneg(x, ntiles));
  const int64_t ub = int64_t(s.unit) * ntiles, ue = ub + ntiles;
  s.next = xe < ue ? xe : ue;
  s.n = int(s.next - x);
  s.k0 = int(x - ub);
  s.slot = -1;
  if (s.n != ntiles) {
    int64_t fb = xb, fe = xe;   // range of the workgroup holding step ub
    if (xb > ub) {
      const int b = wg_of_step(ub, total, G);
      fb = wg_range_start(b, total, G);
      fe = wg_range_start(b + 1, total, G);
    }
    if (fb != ub) {
      s.k0 -= int(fe - ub);
      if (s.k0 < 0) s.k0 += ntiles;
    }
    s.slot = x == xb ? 2 * w : 2 * w + 1;
  }
  return s;
}

// For the merge of unit u: the first workgroup holding part of it, and
// whether that workgroup holds all of it (then nothing is merged).
__host__ __device__ inline int attn_unit_first_wg(int u, int ntiles, int64_t total, int G) {
  return wg_of_step(int64_t(u) * ntiles, total, G);
}
__host__ __device__ inline bool attn_unit_whole(int u, int ntiles, int64_t total, int G) {
  const int b = attn_unit_first_wg(u, ntiles, total, G);
  return wg_range_start(b + 1, total, G) >= int64_t(u + 1) * ntiles;
}
// Partial slot of workgroup b's part of split unit u (b from the first
// workgroup onward while start(b) < end of u): its first segment if its
// range starts inside the unit, else its last.
__host__ __device__ inline int attn_partial_slot(int b, int u, int ntiles, int64_t total, int G) {
  return wg_range_start(b, total, G) >= int64_t(u) * ntiles ? 2 * b : 2 * b + 1;
}

// whether any unit is split (some range boundary falls inside a unit)
inline bool attn_any_split(int ntiles, int64_t total, int G) {
  for (int b = 1; b < G; ++b)
    if (wg_range_start(b, total, G) % ntiles != 0) return true;
  return false;
}

}  // namespace ust
