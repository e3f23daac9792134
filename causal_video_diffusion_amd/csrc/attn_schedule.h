// Integer schedule of the attention: which (head, query tile, key tiles)
// each workgroup computes, and where the partial results of a split unit go.
// Host and device share this code; it touches no memory.
//
// A unit is one (head, 256-query tile); its work is its key tiles
// 0 .. ntiles-1.  With G workgroups and U units:
//  * the first q * G units (q = U / G when U >= G, else 0) run whole, in q
//    rounds: in round k workgroup w takes unit k * G + w from key tile 0, so
//    all workgroups of a round read the same keys at the same time;
//  * the other r = U - q * G units are key-split: their key tiles, unit
//    after unit, form one sequence of r * ntiles steps, cut into G
//    contiguous ranges, one per workgroup (start(b) = b * steps / G).  A
//    range meets one or more units; its part of each unit is a segment, and
//    a unit met by several ranges is merged afterwards from their partial
//    results.
// One workgroup per unit (G = U) is the special case q = 1, r = 0.
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

struct AttnPlan {
  int G;          // workgroups launched
  int ntiles;     // key tiles per unit
  int q;          // whole-unit rounds
  int u0;         // q * G: first key-split unit
  int64_t steps;  // key-split steps: (U - u0) * ntiles
};

// Plan for U units of ntiles key tiles over `requested` (>= 1) workgroups:
// with fewer units than workgroups, all units are key-split over at most one
// workgroup per step.
__host__ __device__ inline AttnPlan attn_plan(int units, int ntiles, int requested) {
  AttnPlan p;
  p.ntiles = ntiles;
  if (units >= requested) {
    p.G = requested;
    p.q = units / requested;
  } else {
    const int64_t all = int64_t(units) * ntiles;
    p.G = int(all < requested ? all : requested);
    p.q = 0;
  }
  p.u0 = p.q * p.G;
  p.steps = int64_t(units - p.u0) * ntiles;
  return p;
}

// first key-split step of workgroup b's range (b <= G)
__host__ __device__ inline int64_t wg_range_start(int b, const AttnPlan& p) {
  return div_nonneg(int64_t(b) * p.steps, p.G);
}

// the workgroup whose range holds key-split step x (0 <= x < steps): the
// largest b with start(b) <= x, which is never an empty range
__host__ __device__ inline int wg_of_step(int64_t x, const AttnPlan& p) {
  int b = int(div_nonneg(x * p.G, p.steps));
  while (b + 1 < p.G && wg_range_start(b + 1, p) <= x) ++b;
  return b;
}

struct AttnSegment {
  int unit;   // (head, query tile) index
  int k0;     // first key tile
  int n;      // key tiles, k0 .. k0 + n - 1
  int slot;   // -1: the whole unit (final output), else the partial slot
};

// Walks one workgroup's segments in execution order: its q whole units,
// then the segments of its key-split range.
struct AttnWalk {
  int k;          // whole-unit rounds done
  int64_t x;      // next key-split step
  int64_t xb, xe; // the workgroup's key-split range
};

__host__ __device__ inline AttnWalk attn_walk(int w, const AttnPlan& p) {
  AttnWalk s;
  s.k = 0;
  s.xb = wg_range_start(w, p);
  s.xe = wg_range_start(w + 1, p);
  s.x = s.xb;
  return s;
}

// Next segment of workgroup w, or false when it has none left.
// Key order inside a split unit: the workgroup holding the unit's first
// step reaches it at the end of its own range, so it takes the unit's last
// key tiles, and the later workgroups take key tiles from 0 upward.  So the
// workgroups on one head read keys near the same position at once, and no
// segment wraps around the unit's key sequence.
// Partial slots: 2w for the range's first segment, 2w + 1 for its last.
__host__ __device__ inline bool attn_next(AttnWalk& s, int w, const AttnPlan& p, AttnSegment& g) {
  const int nt = p.ntiles;
  if (s.k < p.q) {
    g.unit = s.k * p.G + w;
    g.k0 = 0;
    g.n = nt;
    g.slot = -1;
    ++s.k;
    return true;
  }
  if (s.x >= s.xe) return false;
  const int64_t i = div_nonneg(s.x, nt);   // split unit index
  g.unit = p.u0 + int(i);
  const int64_t ub = i * nt, ue = ub + nt;
  const int64_t next = s.xe < ue ? s.xe : ue;
  g.n = int(next - s.x);
  g.k0 = int(s.x - ub);
  g.slot = -1;
  if (g.n != nt) {
    int64_t fb = s.xb, fe = s.xe;   // range of the workgroup holding step ub
    if (s.xb > ub) {
      const int b = wg_of_step(ub, p);
      fb = wg_range_start(b, p);
      fe = wg_range_start(b + 1, p);
    }
    if (fb != ub) {
      g.k0 -= int(fe - ub);
      if (g.k0 < 0) g.k0 += nt;
    }
    g.slot = s.x == s.xb ? 2 * w : 2 * w + 1;
  }
  s.x = next;
  return true;
}

// For the merge of unit u: whether one workgroup computed all of it (then
// nothing is merged), and the workgroups holding its parts.
__host__ __device__ inline bool attn_unit_whole(int u, const AttnPlan& p) {
  if (u < p.u0) return true;
  const int64_t ub = int64_t(u - p.u0) * p.ntiles;
  return wg_range_start(wg_of_step(ub, p) + 1, p) >= ub + p.ntiles;
}
__host__ __device__ inline int attn_unit_first_wg(int u, const AttnPlan& p) {
  return wg_of_step(int64_t(u - p.u0) * p.ntiles, p);
}
// Whether workgroup b (from the first one onward, while start(b) < the
// unit's end) holds a part of split unit u: its range is not empty.
__host__ __device__ inline bool attn_wg_has_part(int b, const AttnPlan& p) {
  return wg_range_start(b + 1, p) > wg_range_start(b, p);
}
__host__ __device__ inline int64_t attn_unit_end(int u, const AttnPlan& p) {
  return int64_t(u - p.u0 + 1) * p.ntiles;
}
// Partial slot of workgroup b's part of split unit u: its first segment if
// its range starts inside the unit, else its last.
__host__ __device__ inline int attn_partial_slot(int b, int u, const AttnPlan& p) {
  return wg_range_start(b, p) >= int64_t(u - p.u0) * p.ntiles ? 2 * b : 2 * b + 1;
}

// whether any unit is split (some non-empty range boundary falls inside a unit)
inline bool attn_any_split(const AttnPlan& p) {
  for (int b = 1; b < p.G; ++b) {
    const int64_t s = wg_range_start(b, p);
    if (s < p.steps && s % p.ntiles != 0) return true;
  }
  return false;
}

}  // namespace ust
