// Host check of the key-split attention schedule (attn_schedule.h), built
// and run by test_host_abi.py on the CPU.  Reads lines "n_units ntiles G"
// (G = the requested workgroup count) and checks, for each:
//  - every (unit, key tile) is computed by exactly one segment;
//  - every segment lies inside its unit's key tiles (no wrap, no overrun)
//    and inside its workgroup's range;
//  - partial slots are < 2 G and used once; a unit is whole (written
//    directly, slot -1) exactly when the merge skips it;
//  - the merge enumerates, for each split unit, exactly the slots that its
//    segments wrote;
//  - the merge is launched exactly when some unit is split.
// Prints "ok" per line, or the first violation and exits 1.
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "../causal_video_diffusion_amd/csrc/attn_schedule.h"

using namespace ust;

static int fail(const char* what, long a, long b, long c) {
  std::printf("FAIL %s (%ld %ld %ld)\n", what, a, b, c);
  return 1;
}

static int check(int units, int ntiles, int requested) {
  const int64_t total = int64_t(units) * ntiles;
  const int G = attn_grid(total, requested);
  if (G < 1 || G > requested) return fail("grid", units, ntiles, requested);
  std::vector<int> cover(size_t(total), 0);
  std::vector<std::set<int>> written(units);   // partial slots per unit
  std::vector<int> whole_writes(units, 0);
  std::set<int> used;
  for (int w = 0; w < G; ++w) {
    const int64_t xb = wg_range_start(w, total, G), xe = wg_range_start(w + 1, total, G);
    if (xe <= xb) return fail("empty range", units, ntiles, w);
    int segs = 0;
    for (int64_t x = xb; x < xe;) {
      const AttnSegment s = attn_segment(x, xb, xe, w, ntiles, total, G);
      if (s.next <= x || s.next > xe) return fail("segment end", w, long(x), long(s.next));
      if (s.unit < 0 || s.unit >= units) return fail("unit", w, s.unit, units);
      if (s.n != s.next - x || s.n < 1) return fail("length", w, s.n, long(s.next - x));
      if (s.k0 < 0 || s.k0 + s.n > ntiles) return fail("key range", w, s.k0, s.n);
      if (int64_t(s.unit) * ntiles > x || int64_t(s.unit + 1) * ntiles < s.next)
        return fail("segment outside its unit", w, s.unit, long(x));
      for (int k = s.k0; k < s.k0 + s.n; ++k) ++cover[size_t(int64_t(s.unit) * ntiles + k)];
      if (s.slot < 0) {
        if (s.n != ntiles) return fail("partial without slot", w, s.unit, s.n);
        ++whole_writes[s.unit];
      } else {
        if (s.slot >= 2 * G) return fail("slot range", w, s.slot, G);
        if (!used.insert(s.slot).second) return fail("slot reused", w, s.slot, s.unit);
        if (s.slot / 2 != w) return fail("slot owner", w, s.slot, s.unit);
        written[s.unit].insert(s.slot);
      }
      x = s.next;
      ++segs;
    }
    if (segs < 1) return fail("no segment", units, ntiles, w);
  }
  for (int64_t i = 0; i < total; ++i)
    if (cover[size_t(i)] != 1) return fail("coverage", long(i / ntiles), long(i % ntiles), cover[size_t(i)]);
  bool any = false;
  for (int u = 0; u < units; ++u) {
    const bool whole = attn_unit_whole(u, ntiles, total, G);
    if (whole != (whole_writes[u] == 1)) return fail("whole flag", u, whole, whole_writes[u]);
    if (whole) {
      if (!written[u].empty()) return fail("whole unit with partials", u, 0, 0);
      continue;
    }
    any = true;
    std::set<int> merged;
    const int64_t ue = int64_t(u + 1) * ntiles;
    for (int b = attn_unit_first_wg(u, ntiles, total, G); b < G && wg_range_start(b, total, G) < ue; ++b)
      merged.insert(attn_partial_slot(b, u, ntiles, total, G));
    if (merged != written[u]) return fail("merge slots", u, long(merged.size()), long(written[u].size()));
  }
  if (any != attn_any_split(ntiles, total, G)) return fail("any split", units, ntiles, G);
  return 0;
}

int main() {
  int units, ntiles, requested, n = 0;
  while (std::scanf("%d %d %d", &units, &ntiles, &requested) == 3) {
    if (check(units, ntiles, requested)) return 1;
    ++n;
  }
  std::printf("ok %d\n", n);
  return n > 0 ? 0 : 1;
}
