// Kernel argument blocks and launchers shared by the host library and the HIP kernels.
// Every struct is passed by value as the kernel argument (kernarg segment), so the
// kernels read layout tables and pointers through the scalar cache.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "plr.h"

namespace plr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte vector

constexpr int kMaxTableSegs = 64;   // explicit segment table carried in kernarg
enum { kXcdOff = 0, kXcdOn = 1 };

// LDS-staged path: depth of each wave's ring of 4 KiB slabs (1 KiB per wave and
// source). The reduce keeps W KiB per stage per wave (4 waves x S x W KiB per
// workgroup: for W = 8, 64 KiB, two workgroups per compute unit's 160 KiB of LDS);
// the copy keeps 1 KiB per stage (16 KiB per workgroup).
constexpr int lds_reduce_stages(int w) { return w <= 4 ? 4 : 2; }
constexpr int kCopyStages = 4;
// Workspace: a header of kWorkspaceHeader bytes (u64 error word at byte 0, u64 ready
// word at byte 8, u64 late counter at byte 16), then uint64 flags[W][nchunks] and their
// check-time mirror uint64 mirror[W][nchunks].
constexpr size_t kWorkspaceHeader = 256;
constexpr int kLateWord = 2;  // u64 header word: count of chunk waits that found a flag missing
constexpr uint64_t kDefaultSpinLimit = 1ull << 20;

// Datapath variants of one launch.
struct Launch {
  uint32_t grid;
  uint32_t block;
  int unroll;
  int stages;
  int datapath;  // PLR_PATH_DIRECT or PLR_PATH_LDS
  uint32_t run;  // consecutive tiles per workgroup
  int xcd;       // XCD-aware workgroup order
  uint32_t lds_bytes;  // LDS reserved per workgroup to cap resident workgroups per CU (0: none)
};

// Notification state of one consuming launch (section 3.2, SNAC "notify").
struct Notify {
  const uint64_t* flags;  // [W][nchunks], or nullptr when the call is not notified
  uint64_t* err;          // sticky error word (workspace header), or nullptr
  const uint64_t* ready;  // set to epoch by the check kernel when every flag had arrived, or nullptr
  const uint64_t* mirror; // per flag: epoch if that flag had arrived at check time (check mode)
  uint64_t epoch;         // a chunk may be consumed once its flags are >= epoch
  uint64_t spin_limit;    // polls before giving up with PLR_ETIMEOUT
};

struct CheckArgs {
  const uint64_t* flags;  // the layout's W*nchunks flags
  uint64_t nflags;
  uint64_t epoch;
  uint64_t* ready;        // receives epoch if every flag is >= epoch, else 0
  uint64_t* mirror;       // per flag: epoch if it is >= epoch, else 0
};
constexpr int kCheckThreads = 1024;  // the check is one workgroup

// Work division shared by reduce and copy: a workgroup consumes a run of whole
// consecutive tiles (a tile is the Atom's step), and tiles_per_chunk consecutive
// tiles of one segment form a chunk, the notification granule whose flags a tile
// waits for.
struct ReduceArgs {
  const u32x4* src[PLR_MAX_WORLD];  // start of the share inside each source
  u32x4* dst;
  uint64_t nvec;        // 16-byte vectors in the share
  uint64_t tile_vecs;   // vectors per tile
  uint32_t ntiles;
  uint32_t tiles_per_chunk;
  uint32_t nchunks;     // flags per source
  uint32_t world;
  uint32_t run;         // consecutive tiles per workgroup
  uint32_t xcd;         // XCD-aware workgroup order
  Notify nt;
};

// Copy segments: all segments of one layout have the same length (seg_len bytes).
// Segment k reads source seg_src[k] at seg_src_off[k] and writes dst at seg_dst_off[k].
// Layouts with more than kMaxTableSegs segments (AllToAll with W > 8) use the
// transposed formula instead of the table: k = s*W + d, src_off = d*slice,
// dst_off = (d*W + s)*slice.
// Variable-length layouts (AllGatherV, at most PLR_MAX_WORLD segments) use the table
// with per-segment lengths and first tiles and chunks instead of one common length.
enum CopyMode : uint32_t { kCopyTable = 0, kCopyTransposed = 1, kCopyVar = 2 };

struct CopyArgs {
  const uint8_t* src[PLR_MAX_WORLD];
  uint8_t* dst;
  uint64_t seg_len;
  uint64_t tile_bytes;
  uint32_t tiles_per_seg;
  uint32_t ntiles;
  uint32_t tiles_per_chunk;
  uint32_t chunks_per_seg;
  uint32_t nchunks;     // chunks of all segments: segment k's chunk j is flag k*chunks_per_seg + j
  uint32_t nseg;
  uint32_t world;
  uint32_t mode;
  uint32_t run;    // consecutive tiles per workgroup
  uint32_t xcd;    // XCD-aware workgroup order
  uint64_t slice;  // kCopyTransposed: bytes per slice
  Notify nt;
  uint32_t seg_src[kMaxTableSegs];
  uint64_t seg_src_off[kMaxTableSegs];
  uint64_t seg_dst_off[kMaxTableSegs];
  // kCopyVar: first tile and first chunk of every segment (nseg + 1 entries, then
  // ~0u in var_tile0), lengths, and the shift of each segment's tiles: tile 0 is that
  // many bytes short, so that every later tile starts on a 128-byte line of the
  // destination (chunks stay whole multiples of the tile size from the segment start)
  uint32_t var_tile0[PLR_MAX_WORLD + 1];
  uint32_t var_chunk0[PLR_MAX_WORLD + 1];
  uint64_t var_len[PLR_MAX_WORLD];
  uint32_t var_shift[PLR_MAX_WORLD];
};

// kernel arguments are limited to 4 KiB
static_assert(sizeof(CopyArgs) <= 4096, "copy kernel arguments exceed 4 KiB");

constexpr int kRankSeg = 1024;  // rows per rank workgroup (one per thread)
constexpr uint32_t kNoDest = 0xFFFFu;

struct CopyVArgs {
  const uint8_t* src[PLR_MAX_WORLD];
  const int32_t* dest[PLR_MAX_WORLD];
  int64_t row_start[PLR_MAX_WORLD + 1];  // prefix of rows_per_src
  uint32_t seg_start[PLR_MAX_WORLD + 1]; // prefix of ceil(rows_per_src / kRankSeg)
  int32_t* seg_count;  // scratch [segments][W]: rows of a segment bound for each destination
  int32_t* seg_out;    // scratch [segments][PLR_MAX_WORLD]: output row of the segment's first row
                       // bound for each destination
  uint8_t* dst;
  int64_t* counts;   // [s][d]
  int64_t* offsets;  // [d][s]
  uint32_t* key;     // scratch, per row: destination << 16 | rank inside its segment and
                     // destination (kNoDest << 16 for a row that has no destination)
  uint32_t* ticket;  // scratch: count of finished rank workgroups (zero between calls)
  uint64_t row_bytes;
  uint64_t tiles_per_row;  // scatter tiles per row (the kernel's tile size)
  uint32_t world;
  uint32_t xcd;      // XCD-aware workgroup order (scatter)
  uint32_t small;    // at most kSmallCounts segment counts: no ticket; the scatter derives
                     // the segments' output rows, counts and offsets from the counts itself
};
constexpr uint32_t kSmallCounts = 256;  // segments x W of the small form (4 per lane of a wave)

// AllReduce of W contributions into W outputs. The share of every output is cut into
// W slices (slice r belongs to rank r) and each slice into tiles.
struct AllReduceArgs {
  const u32x4* src[PLR_MAX_WORLD];
  u32x4* dst[PLR_MAX_WORLD];
  uint64_t slice_vecs;       // 16-byte vectors per slice
  uint64_t tile_vecs;
  uint32_t tiles_per_slice;
  uint32_t ntiles;           // world * tiles_per_slice
  uint32_t world;
  uint32_t run;              // fused: tiles per workgroup
  uint32_t lag;              // composed: a workgroup gathers the tile `lag` below its own
  uint32_t pad;
  Notify nt;                 // composed: per-tile flags (the reducer releases, gatherers acquire)
};

// Latency-path packets: one uint64 per 4-byte payload word, the low 32 bits of the
// epoch in the high half.
struct PackArgs {
  const uint32_t* data[PLR_MAX_WORLD];  // every source's share
  uint64_t* packets[PLR_MAX_WORLD];
  uint64_t nwords;  // payload words per source (a multiple of 4)
  uint32_t first;   // first source of the launch (one source per grid row)
  uint32_t stamp;
};

struct PacketReduceArgs {
  const uint64_t* pk[PLR_MAX_WORLD];  // packets of every source
  uint32_t* dst;
  uint64_t nwords;     // payload words (one packet per source each)
  uint32_t world;
  uint32_t stamp;
  uint64_t* err;
  uint64_t spin_limit;
};

struct NotifyArgs {
  uint64_t* flags;
  uint64_t nflags;  // flags to store, starting at `flags`
  uint64_t epoch;
};

// Measurement events of the calling host thread (plr_set_timing_events), or nulls. The
// first datapath kernel a call launches carries `start` and its last carries `stop`, as
// the dispatch's own start and end timestamps (hipExtLaunchKernel), so that the pair
// times the datapath kernels alone, like a kernel trace.
struct Timing {
  hipEvent_t start;        // start of the first datapath dispatch
  hipEvent_t stop;         // end of the last
  hipEvent_t first_stop;   // end of the first, when it is not also the last (or null)
  hipEvent_t last_start;   // start of the last, when it is not also the first (or null)
};
const Timing& timing();

// Keeps e as the calling thread's last HIP error (plr_last_hip_error); returns PLR_EHIP.
int record_hip_error(hipError_t e);

// Row counts of a variable-length AllToAll: PLR_EINVAL for a negative count (or a
// NULL array), PLR_EUNSUPPORTED for more than 2^31 - 1 rows in all (output rows are
// int32), else PLR_OK. Each count is bounded before it is added, so nothing overflows.
int copy_v_check_rows(int world, const int64_t* rows_per_src);

// Launchers (defined next to their kernels). Return a hipError_t.
hipError_t launch_reduce(const ReduceArgs& a, int dtype, const Launch& l, hipStream_t s);
hipError_t launch_copy(const CopyArgs& a, const Launch& l, hipStream_t s);
hipError_t launch_copy_v(const CopyVArgs& a, hipStream_t s);
hipError_t launch_allreduce(const AllReduceArgs& a, int dtype, const Launch& l, hipStream_t s);
hipError_t launch_pack(const PackArgs& a, uint32_t nsrc, hipStream_t s);
hipError_t launch_reduce_packets(const PacketReduceArgs& a, int dtype, hipStream_t s);
hipError_t launch_notify(const NotifyArgs& a, hipStream_t s);
hipError_t launch_check(const CheckArgs& a, hipStream_t s);

}  // namespace plr
