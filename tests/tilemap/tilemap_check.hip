// Host-side check of the workgroup -> tile placement (bigemm_tilemap.h), run on
// the CPU: no kernel is launched. For grids of every shape up to 48 x 48 tiles
// (and a few larger), CU counts 8 .. 304 and K-block counts around the
// prefetch threshold, it checks that
//  - the tiles' workgroups cover every tile exactly once (grid or padded grid);
//  - the grid is padded exactly when the tiles fill at most half of the CUs and
//    K spans at least kPrefetchMinBlocks blocks, and then to one per CU;
//  - xcd_tiles counts the tiles' workgroups of each XCD (bid % 8), never more
//    than the kernel's one lane per tile allows;
//  - the prefetch workgroups of each XCD hold the indices 0 .. nh - 1 once each,
//    with one nh, and every XCD that holds tiles has at least one;
//  - the units of each XCD (prefetch_units) are distinct, and they are exactly
//    the tile rows and tile columns of the XCD's tiles.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../invariant_gemm_deterministic_amd/csrc/bigemm_tilemap.h"

using namespace bigemm;

static int failures = 0;
#define CHECK(c, ...)                                   \
  do {                                                  \
    if (!(c)) {                                         \
      if (failures++ < 20) {                            \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
        std::printf(__VA_ARGS__);                       \
        std::printf("\n");                              \
      }                                                 \
    }                                                   \
  } while (0)

static void check_case(int tiles_m, int tiles_n, int nkb, int cus) {
  const int ntiles = tiles_m * tiles_n;
  const int grid = prefetch_grid(ntiles, nkb, cus);
  const int slots = cus / kXcds;
  const bool pad = slots >= 2 && 2 * ntiles <= slots * kXcds && nkb >= kPrefetchMinBlocks;
  CHECK(grid == (pad ? slots * kXcds : ntiles), "grid %d for %d tiles, %d blocks, %d CUs", grid, ntiles, nkb, cus);
  // the tiles' workgroups: a bijection onto the tiles; remember each tile's XCD
  std::vector<int> seen(ntiles, 0), xcd_of_t(ntiles, -1);
  for (int bid = 0; bid < ntiles; ++bid) {
    const int t = xcd_order(bid, ntiles);
    CHECK(t >= 0 && t < ntiles, "xcd_order %d of %d", t, ntiles);
    if (t < 0 || t >= ntiles) continue;
    int tm, tn;
    tile_coords(t, tiles_m, tiles_n, tm, tn);
    CHECK(tm >= 0 && tm < tiles_m && tn >= 0 && tn < tiles_n, "tile (%d,%d) of %dx%d", tm, tn, tiles_m, tiles_n);
    if (tm < 0 || tm >= tiles_m || tn < 0 || tn >= tiles_n) continue;
    seen[tm * tiles_n + tn]++;
    xcd_of_t[t] = bid % kXcds;
  }
  for (int i = 0; i < ntiles; ++i) CHECK(seen[i] == 1, "tile %d covered %d times (%dx%d)", i, seen[i], tiles_m, tiles_n);
  if (grid == ntiles) return;
  // the prefetch workgroups: per XCD, indices 0 .. nh - 1 once each
  std::vector<std::vector<int>> hs(kXcds);
  std::vector<int> nhs(kXcds, -1), tiles_on(kXcds, 0);
  for (int bid = 0; bid < ntiles; ++bid) tiles_on[bid % kXcds]++;
  for (int bid = ntiles; bid < grid; ++bid) {
    int h, nh;
    prefetch_helper(bid, grid, ntiles, h, nh);
    const int x = bid % kXcds;
    CHECK(nh >= 1 && h >= 0 && h < nh, "bid %d: index %d of %d", bid, h, nh);
    CHECK(nhs[x] == -1 || nhs[x] == nh, "XCD %d: nh %d and %d", x, nhs[x], nh);
    if (nh < 1 || h < 0 || h >= nh || (nhs[x] != -1 && nhs[x] != nh)) continue;
    nhs[x] = nh;
    hs[x].push_back(h);
  }
  for (int x = 0; x < kXcds; ++x) {
    CHECK(xcd_tiles(x, ntiles) == tiles_on[x], "XCD %d: xcd_tiles %d, tiles %d", x, xcd_tiles(x, ntiles), tiles_on[x]);
    CHECK(tiles_on[x] <= kPrefetchMaxXcdTiles, "XCD %d holds %d tiles", x, tiles_on[x]);
    if (tiles_on[x] > 0) CHECK(nhs[x] >= 1, "XCD %d holds %d tiles and no prefetch workgroup", x, tiles_on[x]);
    if (nhs[x] >= 1) {
      std::vector<int> got(nhs[x], 0);
      for (int h : hs[x]) got[h]++;
      for (int h = 0; h < nhs[x]; ++h) CHECK(got[h] == 1, "XCD %d index %d held %d times", x, h, got[h]);
    }
    if (tiles_on[x] == 0 || tiles_on[x] > kPrefetchMaxXcdTiles) continue;
    // units: distinct, and exactly the rows / columns of the XCD's tiles
    std::vector<int> rows(tiles_on[x]), cols(tiles_on[x]);
    int nrows = 0, ncols = 0;
    prefetch_units(x, ntiles, tiles_m, tiles_n, rows.data(), nrows, cols.data(), ncols);
    std::vector<int> row_used(tiles_m, 0), col_used(tiles_n, 0), row_unit(tiles_m, 0), col_unit(tiles_n, 0);
    for (int b = x; b < ntiles; b += kXcds) {
      int tm, tn;
      tile_of(b, ntiles, tiles_m, tiles_n, tm, tn);
      row_used[tm] = 1;
      col_used[tn] = 1;
    }
    for (int i = 0; i < nrows; ++i) {
      CHECK(rows[i] >= 0 && rows[i] < tiles_m, "XCD %d row unit %d", x, rows[i]);
      if (rows[i] >= 0 && rows[i] < tiles_m) row_unit[rows[i]]++;
    }
    for (int i = 0; i < ncols; ++i) {
      CHECK(cols[i] >= 0 && cols[i] < tiles_n, "XCD %d column unit %d", x, cols[i]);
      if (cols[i] >= 0 && cols[i] < tiles_n) col_unit[cols[i]]++;
    }
    for (int tm = 0; tm < tiles_m; ++tm)
      CHECK(row_unit[tm] == row_used[tm], "XCD %d tile row %d: %d units, used %d", x, tm, row_unit[tm], row_used[tm]);
    for (int tn = 0; tn < tiles_n; ++tn)
      CHECK(col_unit[tn] == col_used[tn], "XCD %d tile column %d: %d units, used %d", x, tn, col_unit[tn],
            col_used[tn]);
  }
}

int main() {
  const int cus_list[] = {8, 16, 24, 80, 128, 256, 304};
  const int nkb_list[] = {1, 8, 31, 32, 33, 64, 256};
  long cases = 0;
  for (int cus : cus_list)
    for (int nkb : nkb_list)
      for (int tm = 1; tm <= 48; ++tm)
        for (int tn = 1; tn <= 48; ++tn, ++cases) check_case(tm, tn, nkb, cus);
  const int big[][2] = {{32, 32}, {8, 112}, {128, 8}, {1, 4096}, {300, 7}};
  for (auto& b : big)
    for (int cus : cus_list) {
      check_case(b[0], b[1], 64, cus);
      ++cases;
    }
  if (failures) {
    std::printf("%d failures in %ld cases\n", failures, cases);
    return 1;
  }
  std::printf("tilemap ok: %ld cases\n", cases);
  return 0;
}
