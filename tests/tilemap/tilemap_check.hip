// Host-side check of the workgroup -> tile placement (bigemm_tilemap.h), run on
// the CPU: no kernel is launched. For grids of every shape up to 48 x 48 tiles
// (and a few larger), CU counts 8 .. 304 and K-block counts around the
// prefetch threshold, it checks that
//  - the tiles' workgroups cover every tile exactly once (grid or padded grid);
//  - the grid is padded exactly when the tiles fill at most half of the CUs and
//    K spans at least kPrefetchMinBlocks blocks, and then to one per CU;
//  - every prefetch workgroup serves a tile whose own workgroup runs on the
//    same XCD (bid % 8), or none when that XCD holds no tile;
//  - the prefetchers of a tile hold ranks 0 .. nrank - 1 once each, with one
//    nrank, so that their blocks rank, rank + nrank, ... cover K once;
//  - on an XCD with at least as many prefetchers as tiles, every tile has one.
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
  // the prefetch workgroups
  std::vector<std::vector<int>> ranks(ntiles);
  std::vector<int> nr(ntiles, -1), tiles_on(kXcds, 0), pf_on(kXcds, 0);
  for (int t = 0; t < ntiles; ++t) tiles_on[xcd_of_t[t]]++;
  for (int bid = ntiles; bid < grid; ++bid) {
    int rank, nrank;
    const int t = prefetch_role(bid, grid, ntiles, rank, nrank);
    const int x = bid % kXcds;
    pf_on[x]++;
    if (tiles_on[x] == 0) {
      CHECK(t == -1, "bid %d on an XCD without tiles got tile %d", bid, t);
      continue;
    }
    CHECK(t >= 0 && t < ntiles, "bid %d: tile %d of %d", bid, t, ntiles);
    if (t < 0 || t >= ntiles) continue;
    CHECK(xcd_of_t[t] == x, "bid %d (XCD %d) serves tile %d on XCD %d", bid, x, t, xcd_of_t[t]);
    CHECK(nrank >= 1 && rank >= 0 && rank < nrank, "bid %d: rank %d of %d", bid, rank, nrank);
    CHECK(nr[t] == -1 || nr[t] == nrank, "tile %d: nrank %d and %d", t, nr[t], nrank);
    if (nrank < 1 || (nr[t] != -1 && nr[t] != nrank)) continue;
    nr[t] = nrank;
    ranks[t].push_back(rank);
  }
  for (int t = 0; t < ntiles; ++t) {
    if (ranks[t].empty()) {
      CHECK(pf_on[xcd_of_t[t]] < tiles_on[xcd_of_t[t]], "tile %d has no prefetcher though its XCD has %d for %d tiles",
            t, pf_on[xcd_of_t[t]], tiles_on[xcd_of_t[t]]);
      continue;
    }
    std::vector<int> got(nr[t], 0);
    for (int r : ranks[t])
      if (r >= 0 && r < nr[t]) got[r]++;
    for (int r = 0; r < nr[t]; ++r) CHECK(got[r] == 1, "tile %d rank %d held %d times", t, r, got[r]);
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
