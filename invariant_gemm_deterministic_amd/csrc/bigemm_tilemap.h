// Workgroup -> tile placement of the bf16 / fp16, MXFP8 and int8 kernels, and
// the prefetch workgroups of the bf16 / fp16 kernel. Placement only: which
// workgroup computes which 128 x 128 tile never changes the arithmetic of any
// output element. Host and device code (the CPU tests check the maps).
#pragma once
#include <hip/hip_runtime.h>

namespace bigemm {

constexpr int kXcds = 8;     // MI355X dispatches workgroups round-robin over 8 XCDs
constexpr int kGroupM = 4;   // tile rows that share W tiles inside one XCD

// Undo the round-robin XCD dispatch so that consecutive tiles land on one XCD
// (its L2 then serves the shared X and W tiles): workgroup bid of a grid of
// nblocks runs tile index xcd_order(bid, nblocks).
__host__ __device__ inline int xcd_order(int bid, int nblocks) {
  const int per = nblocks / kXcds;
  return bid < per * kXcds ? (bid % kXcds) * per + bid / kXcds : bid;
}
// Tile index t -> (tile row, tile column), walking the tiles in groups of
// kGroupM tile-rows so that the XCD's concurrent tiles form a compact block.
__host__ __device__ inline void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = t / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int in = t - group * kGroupM * tiles_n;
  tm = first_m + in % gm;
  tn = in / gm;
}
__host__ __device__ inline void tile_of(int bid, int nblocks, int tiles_m, int tiles_n, int& tm, int& tn) {
  tile_coords(xcd_order(bid, nblocks), tiles_m, tiles_n, tm, tn);
}

// Prefetch workgroups (bf16 / fp16 kernel). With fewer tiles than CUs, each
// tile's workgroup streams its X and W panels alone, at the rate one CU
// sustains against HBM latency, while the other CUs idle. When the tiles fill
// at most half of the CUs and K is long (at least kPrefetchMinBlocks 64-deep K
// blocks), the grid is padded to one workgroup per CU. The extra workgroups of
// an XCD share out the distinct panel blocks its tiles will read (each tile
// row's X lines and each tile column's W lines of one K block, however many of
// the XCD's tiles share them), touch their lines a little ahead of the tiles'
// own workgroups, which then find them in the XCD's L2, and store nothing. The
// tiles, each tile's arithmetic, and so every output byte are the same as with
// a grid of the tiles alone. The condition depends on the tile count, which
// follows M: only which CUs read ahead changes with M, never the work of any
// output element.
constexpr int kPrefetchMinBlocks = 32;
constexpr int kPrefetchMaxXcdTiles = 64;   // one lane per tile of an XCD when the roles are dealt
__host__ __device__ inline int prefetch_grid(int ntiles, int nkb, int cus) {
  const int slots = cus / kXcds;
  if (slots < 2 || 2 * ntiles > slots * kXcds || nkb < kPrefetchMinBlocks ||
      ntiles > kXcds * kPrefetchMaxXcdTiles)
    return ntiles;
  return slots * kXcds;
}

// The tiles of XCD x in a grid whose first ntiles workgroups are the tiles:
// workgroups x, x + kXcds, ... below ntiles (tile_of places each).
__host__ __device__ inline int xcd_tiles(int x, int ntiles) {
  return ntiles > x ? (ntiles - 1 - x) / kXcds + 1 : 0;
}

// A padded grid of nblocks: workgroup bid >= ntiles runs on XCD x = bid % kXcds
// (the same round-robin as the tiles); h is its index among that XCD's
// prefetch workgroups, nh their number (0 <= h < nh).
__host__ __device__ inline void prefetch_helper(int bid, int nblocks, int ntiles, int& h, int& nh) {
  const int x = bid % kXcds;
  const int b0 = ntiles + (x - ntiles % kXcds + kXcds) % kXcds;  // first prefetch workgroup on XCD x
  nh = (nblocks - 1 - b0) / kXcds + 1;
  h = (bid - b0) / kXcds;
}

// The units the prefetch workgroups of XCD x share out: the distinct tile rows
// (X panels) and tile columns (W panels) of its tiles, each listed at the
// first of the XCD's tiles (in workgroup order) that has it. A unit's K block
// kb is work item kb * units + u of its kind, and the XCD's prefetch workgroup
// h takes items h, h + nh, h + 2 nh, ... (host form of the rule the kernel
// applies with one lane per tile).
__host__ inline void prefetch_units(int x, int ntiles, int tiles_m, int tiles_n, int* rows, int& nrows, int* cols,
                                    int& ncols) {
  nrows = 0;
  ncols = 0;
  const int cx = xcd_tiles(x, ntiles);
  for (int i = 0; i < cx; ++i) {
    int tm, tn;
    tile_of(x + kXcds * i, ntiles, tiles_m, tiles_n, tm, tn);
    bool new_row = true, new_col = true;
    for (int j = 0; j < nrows; ++j) new_row = new_row && rows[j] != tm;
    for (int j = 0; j < ncols; ++j) new_col = new_col && cols[j] != tn;
    if (new_row) rows[nrows++] = tm;
    if (new_col) cols[ncols++] = tn;
  }
}

}  // namespace bigemm
