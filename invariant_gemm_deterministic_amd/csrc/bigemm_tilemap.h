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
// blocks), the grid is padded to one workgroup per CU: each extra workgroup
// touches the lines of every nrank-th K block of one tile of its XCD
// (prefetch_role), a little ahead of the tile's own workgroup, which then
// finds them in the XCD's L2. They store nothing; the tiles, each tile's
// arithmetic, and so every output byte are the same as with a grid of the
// tiles alone. The condition depends on the tile count, which follows M: only
// which CUs read ahead changes with M, never the work of any output element.
constexpr int kPrefetchMinBlocks = 32;
__host__ __device__ inline int prefetch_grid(int ntiles, int nkb, int cus) {
  const int slots = cus / kXcds;
  if (slots < 2 || 2 * ntiles > slots * kXcds || nkb < kPrefetchMinBlocks) return ntiles;
  return slots * kXcds;
}

// A grid padded with prefetch workgroups: workgroups 0 .. ntiles - 1 are the
// tiles, placed exactly as in a grid of ntiles (tile_of); workgroup
// bid >= ntiles runs on XCD x = bid % kXcds (the same round-robin) and is
// dealt to one of the cx tiles that XCD holds, round-robin over the XCD's
// prefetch workgroups. Returns the tile's xcd_order index, with rank / nrank
// the workgroup's rank among that tile's prefetchers and their number; -1
// when the XCD holds no tile.
__host__ __device__ inline int prefetch_role(int bid, int nblocks, int ntiles, int& rank, int& nrank) {
  const int x = bid % kXcds;
  const int per = ntiles / kXcds, rem = ntiles - per * kXcds;
  const int cx = per + (x < rem ? 1 : 0);                         // tiles on XCD x
  const int b0 = ntiles + (x - ntiles % kXcds + kXcds) % kXcds;  // first prefetcher on XCD x
  const int hx = (nblocks - 1 - b0) / kXcds + 1;                  // prefetchers on XCD x
  const int h = (bid - b0) / kXcds;                               // this one's index among them
  rank = 0;
  nrank = 0;
  if (cx == 0) return -1;
  const int i = h % cx;
  rank = h / cx;
  nrank = (hx - 1 - i) / cx + 1;
  return i < per ? x * per + i : per * kXcds + x;
}

}  // namespace bigemm
