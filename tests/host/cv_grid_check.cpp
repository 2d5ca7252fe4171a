// CPU check of the variable-length row scatter's work division (copy_v_grid.h): for
// tile counts on both sides of the column cap, in both the small form (one extra
// column that moves no tile) and the ticket form, the tile columns' run loops visit
// every tile of a source exactly once. The cap is lowered so that strided grids are
// small enough to enumerate; the kernel uses the same functions with the real cap.
#include <cstdio>
#include <vector>

#include "copy_v_grid.h"

using namespace plr;

static int check(uint64_t ntiles, uint32_t run, uint32_t cap, bool small) {
  const uint32_t tile_cols = cv_tile_columns(ntiles, run, cap);
  const uint32_t grid = cv_grid_columns(tile_cols, small);
  if (grid != tile_cols + (small ? 1u : 0u)) return 1;
  std::vector<int> seen(ntiles, 0);
  const uint64_t stride = cv_tile_stride(grid, small, run);
  for (uint32_t col = 0; col < grid; ++col) {
    if (small && col == grid - 1) continue;  // the counts-and-offsets column
    for (uint64_t t0 = cv_first_tile(col, run); t0 < ntiles; t0 += stride)
      for (uint64_t t = t0; t < t0 + run && t < ntiles; ++t) seen[t] += 1;
  }
  for (uint64_t t = 0; t < ntiles; ++t)
    if (seen[t] != 1) {
      std::printf("FAIL ntiles=%llu run=%u cap=%u small=%d: tile %llu moved %d times\n",
                  (unsigned long long)ntiles, run, cap, (int)small, (unsigned long long)t, seen[t]);
      return 1;
    }
  return 0;
}

int main() {
  int bad = 0, cases = 0;
  for (uint32_t cap : {1u, 2u, 3u, 7u, 64u})
    for (uint32_t run : {1u, 2u, 4u})
      for (uint64_t ntiles : {0ull, 1ull, 2ull, 5ull, 63ull, 64ull, 65ull, 200ull, 1000ull, 4097ull})
        for (bool small : {false, true}) {
          bad += check(ntiles, run, cap, small);
          ++cases;
        }
  // the real cap: a grid below it covers the tiles in one turn of every column's loop
  if (cv_tile_columns((uint64_t)kCvMaxColumns * 2 + 1, 2, kCvMaxColumns) != kCvMaxColumns) ++bad;
  if (cv_tile_columns(7, 2, kCvMaxColumns) != 4) ++bad;
  std::printf("%s: %d cases\n", bad ? "FAIL" : "ok", cases);
  return bad ? 1 : 0;
}
