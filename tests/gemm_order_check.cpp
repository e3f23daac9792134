// Host check of the GEMM tile order (gemm_order.h), built and run by
// test_host_abi.py on the CPU.  Reads lines "nbm nbn w_bytes" and checks,
// for each grid:
//  - workgroups 0 .. nbm*nbn-1 cover every tile exactly once;
//  - each XCD (workgroup b on XCD b % 8) gets a contiguous run of tile
//    indices, the first ntile % 8 XCDs one more than the others;
//  - the row-major order applies exactly when the grid fits in one round of
//    the chip or the weight fits in one XCD's L2;
//  - in the grouped order, the tiles an XCD runs at one time (32 consecutive
//    workgroups of that XCD), where they lie in groups of kGroupRows full
//    row blocks, span at most 2 kGroupRows row blocks and 32 / kGroupRows +
//    2 column blocks (one group's compact block, or the ends of two): not a
//    run along one row's columns.
// Then, for extra workgroups past a launch's tiles (xcd_range_pos), that
// each range maps onto its positions once, in contiguous per-XCD runs.
// Prints "ok <count>", or the first violation and exits 1.
#include <cstdio>
#include <set>
#include <vector>

#include "../causal_video_diffusion_amd/csrc/gemm_order.h"

using namespace ust;

static int fail(const char* what, long a, long b, long c) {
  std::printf("FAIL %s (%ld %ld %ld)\n", what, a, b, c);
  return 1;
}

static int check(int nbm, int nbn, long long w_bytes) {
  const int ntile = nbm * nbn;
  const bool row_major = ntile <= kChipCUs || w_bytes <= kL2Bytes;
  std::vector<int> seen(size_t(ntile), 0);
  for (int b = 0; b < ntile; ++b) {
    const GemmTile t = gemm_tile(b, nbm, nbn, w_bytes);
    if (t.m_blk < 0 || t.m_blk >= nbm || t.n_blk < 0 || t.n_blk >= nbn)
      return fail("tile outside the grid", b, t.m_blk, t.n_blk);
    if (seen[size_t(t.m_blk) * nbn + t.n_blk]++) return fail("tile computed twice", b, t.m_blk, t.n_blk);
  }
  // per XCD: the sequence of tiles its workgroups take, in dispatch order
  for (int x = 0; x < 8; ++x) {
    const int share = ntile / 8 + (x < ntile % 8 ? 1 : 0);
    int count = 0;
    std::vector<GemmTile> run;
    for (int b = x; b < ntile; b += 8) {
      run.push_back(gemm_tile(b, nbm, nbn, w_bytes));
      ++count;
    }
    if (count != share) return fail("XCD share", x, count, share);
    if (row_major) {
      // consecutive row-major indices
      for (size_t i = 1; i < run.size(); ++i) {
        const long a = long(run[i - 1].m_blk) * nbn + run[i - 1].n_blk;
        const long c = long(run[i].m_blk) * nbn + run[i].n_blk;
        if (c != a + 1) return fail("row-major run not contiguous", x, a, c);
      }
    } else {
      const int full_rows = nbm / kGroupRows * kGroupRows;   // rows in full groups
      for (size_t i = 0; i + 32 <= run.size(); i += 32) {
        std::set<int> rows, cols;
        bool in_full = true;
        for (size_t k = i; k < i + 32; ++k) {
          rows.insert(run[k].m_blk);
          cols.insert(run[k].n_blk);
          in_full = in_full && run[k].m_blk < full_rows;
        }
        if (in_full && (int(rows.size()) > 2 * kGroupRows || int(cols.size()) > 32 / kGroupRows + 2))
          return fail("grouped block not compact", x, long(rows.size()), long(cols.size()));
      }
    }
  }
  return 0;
}

// Extra workgroups [lo, hi) of a launch (xcd_range_pos): positions 0 ..
// hi-lo-1 each exactly once, and each XCD's workgroups, in dispatch order,
// on consecutive positions, the runs following XCD order.
static int check_range(int lo, int hi) {
  std::vector<int> seen(size_t(hi - lo), 0);
  for (int b = lo; b < hi; ++b) {
    const int p = xcd_range_pos(b, lo, hi);
    if (p < 0 || p >= hi - lo) return fail("range position outside", lo, hi, b);
    if (seen[size_t(p)]++) return fail("range position taken twice", lo, hi, b);
  }
  int next = 0;
  for (int x = 0; x < 8; ++x)
    for (int b = lo; b < hi; ++b)
      if ((b & 7) == x) {
        if (xcd_range_pos(b, lo, hi) != next) return fail("range run not contiguous", lo, hi, b);
        ++next;
      }
  return 0;
}

int main() {
  int nbm, nbn;
  long long w_bytes;
  int count = 0;
  while (std::scanf("%d %d %lld", &nbm, &nbn, &w_bytes) == 3) {
    if (check(nbm, nbn, w_bytes)) return 1;
    ++count;
  }
  const int los[] = {0, 1, 3, 7, 8, 9, 148, 228, 684};
  for (int lo : los)
    for (int n = 1; n <= 70; ++n) {
      if (check_range(lo, lo + n)) return 1;
      ++count;
    }
  for (int lo : los)
    for (int n : {225, 450, 900, 1001}) {
      if (check_range(lo, lo + n)) return 1;
      ++count;
    }
  std::printf("ok %d\n", count);
  return 0;
}
