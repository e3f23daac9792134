// Tile order of the pipelined GEMM: which output tile a workgroup computes,
// and the order of the extra workgroups a launch may carry beyond its
// tiles.  Host and device share this code; it touches no memory.
//
// Workgroups are dealt to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8), so XCD x receives workgroups x, x + 8, x + 16, ...; each XCD is
// given a contiguous run of tile indices, the first ntile % 8 XCDs one tile
// more than the rest.  A tile index becomes a (row block, column block)
// pair in one of two orders:
//  * row-major, when the tiles fit in one round of the chip or the weight
//    (N x K bf16) fits in one XCD's L2: the tiles an XCD runs at one time
//    share their rows of X;
//  * grouped, otherwise: the indices run over groups of kGroupRows row
//    blocks, column by column within a group, so the tiles an XCD runs at
//    one time form a compact block (4 x 8 for 32 CUs) whose rows of X and
//    columns of W its L2 serves to several tiles each.  The last group may
//    hold fewer row blocks.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace ust {

constexpr int kChipCUs = 256;                     // compute units of the part
constexpr int kGroupRows = 4;                     // row blocks per group of the grouped order
constexpr int64_t kL2Bytes = int64_t(4) << 20;    // L2 of one XCD

struct GemmTile {
  int m_blk, n_blk;
};

// tile of workgroup b (0 <= b < nbm * nbn) for an nbm x nbn grid of tiles
// and a weight of w_bytes
__host__ __device__ inline GemmTile gemm_tile(int b, int nbm, int nbn, int64_t w_bytes) {
  const int ntile = nbm * nbn;
  const int xcd = b & 7, q = ntile >> 3, r = ntile & 7;
  const int tile = xcd * q + (xcd < r ? xcd : r) + (b >> 3);
  if (ntile <= kChipCUs || w_bytes <= kL2Bytes) return GemmTile{tile / nbn, tile % nbn};
  const int grp = tile / (kGroupRows * nbn), first = grp * kGroupRows;
  const int rows = nbm - first < kGroupRows ? nbm - first : kGroupRows;
  const int local = tile - grp * kGroupRows * nbn;
  return GemmTile{first + local % rows, local / rows};
}

// Position of workgroup b in the range [lo, hi) of a grid (lo <= b < hi)
// when the range's workgroups are dealt to the XCDs in contiguous runs of
// positions: XCD x's workgroups of the range, in dispatch order, take the
// next positions of run x, and run x follows runs 0 .. x-1.
__host__ __device__ inline int xcd_range_pos(int b, int lo, int hi) {
  const int x = b & 7;
  int start = 0;
  for (int y = 0; y < x; ++y) {
    const int first = lo + ((y - lo) % 8 + 8) % 8;   // the range's first workgroup on XCD y
    start += first < hi ? (hi - 1 - first) / 8 + 1 : 0;
  }
  const int firstx = lo + ((x - lo) % 8 + 8) % 8;
  return start + (b - firstx) / 8;
}

}  // namespace ust
