// Work division of the variable-length row scatter, shared by its host launcher and its
// kernel. Plain C++ with no HIP types, so that a CPU test can compile it on its own and
// check that every tile is moved exactly once, the capped grids included.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define PLR_HD __host__ __device__
#else
#define PLR_HD
#endif

namespace plr {

constexpr uint32_t kCvMaxColumns = 1u << 22;  // tile columns of one scatter launch at most

// Columns of the scatter grid that move tiles: one per run of `run` tiles of the source
// with the most tiles, at least 1 and at most `cap` (past that every column strides).
PLR_HD inline uint32_t cv_tile_columns(uint64_t most_tiles, uint32_t run, uint32_t cap) {
  const uint64_t runs = (most_tiles + run - 1) / run;
  return (uint32_t)(runs < 1 ? 1 : (runs > cap ? cap : runs));
}

// The grid's columns: the tile columns, plus, in the small form, one last column that
// writes counts and offsets and moves no tile.
PLR_HD inline uint32_t cv_grid_columns(uint32_t tile_cols, bool small) { return tile_cols + (small ? 1u : 0u); }

// Tile column c starts at tile c * run and steps by the tile columns' runs, so the
// columns together visit every run once whatever the cap.
PLR_HD inline uint64_t cv_first_tile(uint32_t col, uint32_t run) { return (uint64_t)col * run; }
PLR_HD inline uint64_t cv_tile_stride(uint32_t grid_cols, bool small, uint32_t run) {
  return (uint64_t)(grid_cols - (small ? 1u : 0u)) * run;
}

}  // namespace plr
