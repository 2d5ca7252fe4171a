// Host-side compiled layout: the segment and chunk table plus the resolved policy.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "plr.h"

struct plr_layout {
  struct Seg {
    int src;
    uint64_t src_off;
    uint64_t dst_off;
    uint64_t len;
  };

  plr_op op;
  plr_dtype dtype;
  int world;
  int rank;
  uint64_t bytes_per_src;
  plr_layout_kind in_kind, out_kind;

  // compiled table (section 3.1 "Layouts"): reduce has one segment per source, all
  // with the share length; copy has W or W*W segments of one common length
  std::vector<Seg> segs;
  uint64_t seg_len;
  uint64_t src_bytes;  // the most bytes any one source contributes: the policy's regime
  uint64_t dst_bytes;
  bool table_fits;  // copy: the table is carried in the kernel arguments
  bool var_segs;    // copy: segments of different lengths (AllGatherV)

  // work and notification granules: a tile is what one workgroup consumes per
  // step; a chunk (a whole number of tiles of one segment) is what one flag per
  // source announces (section 3.2 "SNAC")
  uint64_t tile_bytes;       // per source (reduce) / per segment piece (copy)
  uint64_t chunk_bytes;
  uint32_t tiles_per_seg;
  uint32_t tiles_per_chunk;
  uint32_t chunks_per_seg;
  uint32_t ntiles;           // reduce: tiles of the share; copy: tiles of all segments
  uint32_t nchunks;          // reduce: chunks of the share; copy: chunks of all segments
  // un-notified calls wait for no chunk, so a reduce may launch them with a tile and
  // workgroup size of their own; every other layout uses the shape above for both
  uint64_t plain_tile_bytes;
  uint32_t plain_ntiles;
  int plain_block;
  // copy: first tile and first chunk of every segment (nseg + 1 entries; with equal
  // segments k * tiles_per_seg and k * chunks_per_seg), and first flag of every
  // source (W + 1 entries): segments go source by source
  std::vector<uint32_t> seg_tile0, seg_chunk0, src_flag0;
  std::vector<uint32_t> seg_shift;  // variable-length copy: bytes tile 0 of a segment is short

  // resolved policy (section 4.2 "Codesign Policies and Tuning")
  int workgroups;  // explicit grid size, or 0
  int run;           // tiles per workgroup when workgroups is 0
  int run_notified;  // the same for notified calls (each workgroup pays one acquire per chunk)
  int notify_mode;   // PLR_NOTIFY_CHUNKS or PLR_NOTIFY_CHECK
  int xcd_order;     // kXcdOff or kXcdOn
  int lag;           // allreduce, composed: tiles between a workgroup's reduction and its gather
  int block;
  int unroll;
  int stages;
  int datapath;
  int wgs_per_cu;        // resident-workgroup cap of the direct-path launches, 0 = none
  uint32_t lds_reserve;  // LDS bytes each such launch reserves for the cap
  uint64_t spin_limit;

  uint64_t epoch;  // section 4.3 "Epoch Bookkeeping"
};

namespace plr {
size_t elem_bytes(plr_dtype t);

// Chunk flags of a notified layout. Reduce: flags[W][nchunks], one per source and chunk
// of the share. Copy: one per chunk of every segment, in segment order (segment k's
// chunk j is flag seg_chunk0[k] + j); segments are listed source by source, so source
// s's flags are one contiguous range.
inline uint64_t nflags(const plr_layout* L) {
  return L->op == PLR_OP_COPY ? (uint64_t)L->nchunks : (uint64_t)L->world * L->nchunks;
}
// First flag and flag count of source s (reduce: its row of the flag matrix).
inline void src_flags(const plr_layout* L, int s, uint64_t* first, uint64_t* count) {
  if (L->op == PLR_OP_COPY) {
    *first = L->src_flag0[s];
    *count = (uint64_t)L->src_flag0[s + 1] - L->src_flag0[s];
  } else {
    *first = (uint64_t)s * L->nchunks;
    *count = L->nchunks;
  }
}
}
