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
  uint64_t dst_bytes;
  bool table_fits;  // copy: the table is carried in the kernel arguments

  // chunking (section 3.2 "SNAC": the notification granule)
  uint64_t chunk_bytes;      // per source (reduce) / per segment piece (copy)
  uint32_t chunks_per_seg;   // copy only
  uint32_t nchunks;

  // resolved policy (section 4.2 "Codesign Policies and Tuning")
  int workgroups;  // 0 = sized at launch from the device's compute-unit count
  int wg_per_cu;   // used when workgroups == 0
  int block;
  int unroll;
  int stages;
  int datapath;
  uint64_t spin_limit;

  uint64_t epoch;  // section 4.3 "Epoch Bookkeeping"
};

namespace plr {
size_t elem_bytes(plr_dtype t);
}
