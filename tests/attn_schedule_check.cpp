// Host check of the attention schedule (attn_schedule.h), built and run by
// test_host_abi.py on the CPU.  Reads lines "n_units ntiles G" (G = the
// requested workgroup count) and checks, for each plan:
//  - every (unit, key tile) is computed by exactly one segment;
//  - every segment lies inside its unit's key tiles (no wrap, no overrun);
//  - whole-unit rounds come first and give round k's unit k * G + w to
//    workgroup w; key-split segments lie in their workgroup's range;
//  - partial slots are < 2 G, belong to their workgroup and are used once;
//    a unit is whole (written directly, slot -1) exactly when the merge
//    skips it;
//  - the merge enumerates, for each split unit, exactly the slots that its
//    segments wrote;
//  - the merge is launched exactly when some unit is split.
// Prints "ok <count>", or the first violation and exits 1.
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
  const AttnPlan p = attn_plan(units, ntiles, requested);
  if (p.G < 1 || p.G > requested) return fail("grid", units, ntiles, requested);
  if (p.u0 != p.q * p.G || p.u0 > units || (units >= requested && units - p.u0 >= p.G))
    return fail("rounds", units, p.q, p.G);
  if (p.steps != int64_t(units - p.u0) * ntiles) return fail("steps", units, ntiles, long(p.steps));
  std::vector<int> cover(size_t(units) * ntiles, 0);
  std::vector<std::set<int>> written(units);   // partial slots per unit
  std::vector<int> whole_writes(units, 0);
  std::set<int> used;
  for (int w = 0; w < p.G; ++w) {
    AttnWalk s = attn_walk(w, p);
    AttnSegment g;
    int k = 0;
    int64_t x = s.xb;
    while (attn_next(s, w, p, g)) {
      if (g.unit < 0 || g.unit >= units) return fail("unit", w, g.unit, units);
      if (g.n < 1 || g.k0 < 0 || g.k0 + g.n > ntiles) return fail("key range", w, g.k0, g.n);
      if (k < p.q) {
        if (g.unit != k * p.G + w || g.k0 != 0 || g.n != ntiles || g.slot != -1)
          return fail("whole round", w, k, g.unit);
        ++k;
      } else {
        // a key-split segment: steps [x, x + n) of this workgroup's range
        if (g.unit < p.u0) return fail("split unit in rounds", w, g.unit, p.u0);
        const int64_t ub = int64_t(g.unit - p.u0) * ntiles;
        if (x < ub || x + g.n > ub + ntiles || x + g.n > s.xe)
          return fail("segment outside range", w, g.unit, long(x));
        x += g.n;
      }
      for (int t = g.k0; t < g.k0 + g.n; ++t) ++cover[size_t(g.unit) * ntiles + t];
      if (g.slot < 0) {
        if (g.n != ntiles) return fail("partial without slot", w, g.unit, g.n);
        ++whole_writes[g.unit];
      } else {
        if (g.slot >= 2 * p.G) return fail("slot range", w, g.slot, p.G);
        if (!used.insert(g.slot).second) return fail("slot reused", w, g.slot, g.unit);
        if (g.slot / 2 != w) return fail("slot owner", w, g.slot, g.unit);
        written[g.unit].insert(g.slot);
      }
    }
    if (k != p.q || x != s.xe) return fail("walk incomplete", w, k, long(x));
  }
  for (size_t i = 0; i < cover.size(); ++i)
    if (cover[i] != 1) return fail("coverage", long(i / ntiles), long(i % ntiles), cover[i]);
  bool any = false;
  for (int u = 0; u < units; ++u) {
    const bool whole = attn_unit_whole(u, p);
    if (whole != (whole_writes[u] == 1)) return fail("whole flag", u, whole, whole_writes[u]);
    if (whole) {
      if (!written[u].empty()) return fail("whole unit with partials", u, 0, 0);
      continue;
    }
    any = true;
    std::set<int> merged;
    const int64_t ue = attn_unit_end(u, p);
    for (int b = attn_unit_first_wg(u, p); b < p.G && wg_range_start(b, p) < ue; ++b)
      if (attn_wg_has_part(b, p)) merged.insert(attn_partial_slot(b, u, p));
    if (merged != written[u]) return fail("merge slots", u, long(merged.size()), long(written[u].size()));
  }
  if (any != attn_any_split(p)) return fail("any split", units, ntiles, p.G);
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
