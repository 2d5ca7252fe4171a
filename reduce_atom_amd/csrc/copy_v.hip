// Variable-length AllToAll packing (MoE dispatch shape).
//
// Purlin paper, appendix C.4 "Variable-Length Collectives" (partition sizes are
// passed at run time) and section 4 (partition offsets come from prefix sums).
// Output rows are packed per destination, in source then row order:
//   kernel 1 (one workgroup per 1024-row segment of a source): for every row, its
//            destination and its rank among the earlier rows of its segment bound for
//            the same destination (wave ballots plus a workgroup-wide exclusive scan),
//            packed into one key, and the segment's counts; the last of those
//            workgroups scans the segments: counts[s][d], offsets[d][s] (an exclusive
//            scan in destination-major order) and, per segment and destination, the
//            output row of the segment's first row bound there;
//   kernel 2 (row tiles, one per workgroup step): moves every row with 16-byte loads
//            and stores to that segment row plus the row's rank.
// Calls with at most 256 segment counts (segments x W) skip the last workgroup's
// scan: kernel 1 stops at the counts, and kernel 2 derives each tile's segment row from
// them with one wave sum and writes counts and offsets from one extra workgroup; that
// removes a chain of dependent global round trips (release, ticket, acquire, loads)
// from every such call.
#include <algorithm>

#include "copy_v_grid.h"
#include "device_common.h"

namespace plr {

constexpr int kRankThreads = kRankSeg;
constexpr int kRankWaves = kRankThreads / 64;
constexpr uint32_t kCountLds = 8192;  // segment counts the last rank workgroup stages in LDS

// Kernel 1: one workgroup per segment of kRankSeg consecutive rows of one source, one
// row per thread. A wave ballot per destination gives each row its rank among the
// lower lanes bound for the same destination, and per-wave totals in LDS the rank
// across waves: the row's rank inside its segment. The segment's per-destination
// counts go to scratch. The last workgroup to finish (a ticket counter in scratch,
// acquire-release at agent scope, left at zero again) loads all segment counts at once
// (into LDS when they fit) and scans them into counts[s][d], offsets[d][s] and
// seg_out[segment][d] = offsets[d][s] + the rows of the same source's earlier
// segments bound for d.
__global__ void __launch_bounds__(kRankThreads) k_copy_v_rank(const CopyVArgs a) {
  __shared__ int32_t wave_cnt[kRankWaves][PLR_MAX_WORLD];
  __shared__ int64_t tot[PLR_MAX_WORLD * PLR_MAX_WORLD];
  __shared__ int64_t off[PLR_MAX_WORLD * PLR_MAX_WORLD];
  __shared__ int32_t cnt_lds[kCountLds];
  __shared__ int last;

  const int W = (int)a.world;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const uint32_t seg = blockIdx.x;
  // With no rows at all the launch still has one workgroup, which owns no segment and
  // only writes the (zero) counts and offsets.
  const bool has_seg = seg < a.seg_start[W];
  int s = 0;
  if (has_seg)
    while (seg >= a.seg_start[s + 1]) ++s;
  const int64_t i = has_seg ? (int64_t)(seg - a.seg_start[s]) * kRankSeg + t : 0;  // row within source s
  const int64_t rows = has_seg ? a.row_start[s + 1] - a.row_start[s] : 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes < this one

  const int d = (i < rows) ? a.dest[s][i] : -1;
  int in_wave = 0;  // rows of lower lanes in this wave bound for d
#pragma unroll
  for (int dd = 0; dd < PLR_MAX_WORLD; ++dd) {
    if (dd < W) {
      const uint64_t m = __ballot(d == dd);
      if (lane == 0) wave_cnt[wave][dd] = __popcll(m);
      if (d == dd) in_wave = __popcll(m & below);
    }
  }
  __syncthreads();
  if (i < rows) {
    uint32_t key = kNoDest << 16;  // no destination: the row is dropped
    if (d >= 0 && d < W) {
      int r = in_wave;
      for (int w2 = 0; w2 < wave; ++w2) r += wave_cnt[w2][d];
      key = ((uint32_t)d << 16) | (uint32_t)r;
    }
    a.key[a.row_start[s] + i] = key;
  }
  if (has_seg && t < W) {
    int c = 0;
    for (int w2 = 0; w2 < kRankWaves; ++w2) c += wave_cnt[w2][t];
    a.seg_count[(uint64_t)seg * W + t] = c;
  }

  // small form: the scatter kernel reads the segment counts itself
  if (a.small) return;
  // ticket: the last workgroup sees every segment's counts
  __syncthreads();
  if (t == 0) {
    const uint32_t done = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = (done == gridDim.x - 1);
  }
  __syncthreads();
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // every segment count in one round of loads, staged in LDS when they fit
  const uint64_t nsc = (uint64_t)a.seg_start[W] * W;
  const bool staged = nsc <= kCountLds;
  if (staged)
    for (uint64_t k = t; k < nsc; k += kRankThreads)
      cnt_lds[k] = __hip_atomic_load(a.seg_count + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  auto seg_cnt = [&](uint64_t k) -> int32_t {
    return staged ? cnt_lds[k] : __hip_atomic_load(a.seg_count + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  const int WW = W * W;
  if (t < WW) {  // thread (s2, d2): source s2's rows bound for d2
    const int s2 = t / W, d2 = t - s2 * W;
    int64_t run = 0;
    for (uint32_t g = a.seg_start[s2]; g < a.seg_start[s2 + 1]; ++g) run += seg_cnt((uint64_t)g * W + d2);
    tot[t] = run;
    a.counts[t] = run;  // counts[s2][d2]
  }
  __syncthreads();
  if (t < WW) {
    // block (d, s): every block of a smaller destination, then the blocks of
    // smaller sources for the same destination
    const int d3 = t / W, s3 = t - d3 * W;
    int64_t o = 0;
    for (int dd = 0; dd < d3; ++dd)
      for (int ss = 0; ss < W; ++ss) o += tot[ss * W + dd];
    for (int ss = 0; ss < s3; ++ss) o += tot[ss * W + d3];
    off[t] = o;
    a.offsets[t] = o;  // offsets[d3][s3]
  }
  __syncthreads();
  if (t < WW) {  // thread (s2, d2) again: first output row of each segment's d2 rows
    const int s2 = t / W, d2 = t - s2 * W;
    int64_t run = off[d2 * W + s2];
    for (uint32_t g = a.seg_start[s2]; g < a.seg_start[s2 + 1]; ++g) {
      a.seg_out[(uint64_t)g * PLR_MAX_WORLD + d2] = (int32_t)run;
      run += seg_cnt((uint64_t)g * W + d2);
    }
  }
  if (t == 0) __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Kernel 2 cuts every row into tiles of Shape::kTile bytes (the last tile of a row may be
// shorter); a workgroup of Shape::kThreads lanes moves Shape::kRun consecutive tiles of one
// source (grid row y = source y), one 16-byte vector per lane per step, so that the
// chip holds many short workgroups with their loads in flight, as the copy kernel
// does. A tile's source address and the locations of its row's key and segment table
// depend only on the row, so a workgroup issues the data loads of its whole run, then
// the keys and tables, computes each output row (the segment table's entry for the
// key's destination plus the key's rank, with no second dependent load) and stores
// last.
// Two shapes, chosen by the row size: rows over 1 KiB take 2 KiB tiles of 128 lanes in
// runs of 2 (measured on 8 x 4096 rows of 14,336 B: 153-155 us, against 156-158 us for
// runs of 3 or 4 and 160 us for 4 KiB tiles); rows of at most 1 KiB take 1 KiB tiles of
// 64 lanes in runs of 4 (8 x 4096 rows of 64 B: 15-17 us against 22-23 us), so that a
// small row does not leave most lanes of a large workgroup idle.
template <int THREADS, int TILE, int RUN>
struct CvShape {
  static constexpr int kThreads = THREADS;
  static constexpr uint64_t kTile = TILE;
  static constexpr uint32_t kRun = RUN;
  static constexpr int kVecs = TILE / 16 / THREADS;  // vectors per lane per tile
  static_assert(TILE % (16 * THREADS) == 0, "a tile is whole vectors of every lane");
};
using CvLarge = CvShape<128, 2048, 2>;
using CvSmall = CvShape<64, 1024, 4>;
constexpr uint64_t kCvSmallRow = 1024;  // rows of at most this many bytes take CvSmall

// Small form (segments x W <= kSmallCounts): kernel 1 stopped after the segment counts.
// Lane k of every wave keeps CPL of them (counts k*CPL .. k*CPL+CPL-1; count c is
// segment c / W, destination c % W); the output row of a tile's first row of segment g
// bound for d is the sum of the counts of every smaller destination plus those of d in
// earlier segments (segments go source by source, so that is every row placed before
// it): one wave sum per tile. One extra workgroup, with no tiles, writes counts and
// offsets from the same counts, so that no tile waits for it.
// Sum over the 64 lanes of a wave (all active), returned to every lane: DPP moves add
// within quads, then across each row of 16 (rotations), then rows 0..3 into lane 63 (row
// broadcasts; only lane 63 ends with the whole sum), which is then read as a scalar.
// Measured 1 us faster per AllToAllV than the LDS-routed shuffle form.
template <int CTRL>
__device__ __forceinline__ int32_t dpp_mov(int32_t x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ int32_t wave_sum(int32_t x) {
  x += dpp_mov<0xb1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4e>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x124>(x);  // row_ror:4
  x += dpp_mov<0x128>(x);  // row_ror:8: every lane holds its row's sum
  x += dpp_mov<0x142>(x);  // row_bcast:15
  x += dpp_mov<0x143>(x);  // row_bcast:31
  return __builtin_amdgcn_readlane(x, 63);
}

template <int CPL>
__device__ void small_counts_and_offsets(const CopyVArgs& a, const int32_t (&my_cnt)[CPL]) {
  __shared__ int32_t cnt[64 * CPL];
  __shared__ int32_t tot[PLR_MAX_WORLD * PLR_MAX_WORLD];
  const uint32_t W = a.world, WW = W * W;
  if (threadIdx.x < 64)
#pragma unroll
    for (int j = 0; j < CPL; ++j) cnt[threadIdx.x * CPL + j] = my_cnt[j];  // zero past the counts
  __syncthreads();
  for (uint32_t q = threadIdx.x; q < WW; q += blockDim.x) {  // q = (s, d): rows of s bound for d
    const uint32_t s = q / W, d = q - s * W;
    int32_t c = 0;
    for (uint32_t g = a.seg_start[s]; g < a.seg_start[s + 1]; ++g) c += cnt[g * W + d];
    tot[q] = c;
    a.counts[q] = c;
  }
  __syncthreads();
  for (uint32_t q = threadIdx.x; q < WW; q += blockDim.x) {
    // q = (d, s): every row bound for a smaller destination, then the rows bound for d
    // from smaller sources
    const uint32_t d = q / W, s = q - d * W;
    int64_t o = 0;
    for (uint32_t dd = 0; dd < d; ++dd)
      for (uint32_t ss = 0; ss < W; ++ss) o += tot[ss * W + dd];
    for (uint32_t ss = 0; ss < s; ++ss) o += tot[ss * W + d];
    a.offsets[q] = o;
  }
}

// CPL = counts per lane of the small form; 0 = the ticket form (segment table).
template <int CPL, class Shape>
__global__ void __launch_bounds__(Shape::kThreads) k_copy_v_scatter(const CopyVArgs a) {
  constexpr int kCvThreads = Shape::kThreads;
  constexpr uint64_t kCvTileBytes = Shape::kTile;
  constexpr uint32_t kCvRun = Shape::kRun;
  constexpr int kCvVecs = Shape::kVecs;
  constexpr int C = CPL > 0 ? CPL : 1;
  const uint32_t W = a.world;
  int32_t my_cnt[C];
  uint32_t my_seg[C], my_dest[C];
  if (CPL > 0) {
    const uint32_t n = a.seg_start[W] * W, k0 = __lane_id() * CPL;
    if (CPL == 4 && k0 + 3 < n) {  // one 16-byte load (the count region is 256-byte aligned)
      const int4 v = *reinterpret_cast<const int4*>(a.seg_count + k0);
      my_cnt[0] = v.x, my_cnt[1 % C] = v.y, my_cnt[2 % C] = v.z, my_cnt[3 % C] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < C; ++j) my_cnt[j] = k0 + j < n ? a.seg_count[k0 + j] : 0;
    }
#pragma unroll
    for (int j = 0; j < C; ++j) {
      my_seg[j] = (k0 + j) / W;
      my_dest[j] = k0 + j - my_seg[j] * W;
    }
    if (blockIdx.x == gridDim.x - 1) {  // the extra column: no tiles
      if (blockIdx.y == 0) small_counts_and_offsets<C>(a, my_cnt);
      return;
    }
  }
  // Written by kernel 1 and only read here, and the same for every lane of a tile:
  // read through the constant address space so that they are scalar loads, which
  // leave the vector memory path to the row's data.
  const PLR_CONST uint32_t* key_of = (const PLR_CONST uint32_t*)a.key;
  const PLR_CONST int32_t* seg_out = (const PLR_CONST int32_t*)a.seg_out;
  // grid row s moves source s's rows: no search for the source of a tile
  const uint32_t s = blockIdx.y;
  const int64_t r0 = a.row_start[s];
  const uint64_t ntiles = (uint64_t)(a.row_start[s + 1] - r0) * a.tiles_per_row;
  const uint8_t* src_s = a.src[s];
  const uint32_t seg0 = a.seg_start[s];
  // the small form's last column moved no tile and is not part of the stride
  const uint64_t stride = cv_tile_stride(gridDim.x, CPL > 0, kCvRun);
  for (uint64_t t0 = cv_first_tile(logical_block(a.xcd), kCvRun); t0 < ntiles; t0 += stride) {
    const uint32_t m = (uint32_t)min<uint64_t>(kCvRun, ntiles - t0);  // tiles of this run
    // Every data load of the run is issued first, then every key and segment table, and
    // the stores come last: no store of one tile sits between the next tile's loads or
    // its output-row arithmetic and the registers they reuse (which would make them wait
    // for the store), and all of the run's bytes are in flight at once.
    // Straight-line code for every run: a tile past the run's end repeats its last tile's
    // row with no vectors, so it loads and stores nothing.
    uint64_t row[kCvRun], b0[kCvRun], nv[kCvRun];
    u32x4 x[kCvRun][kCvVecs];
#pragma unroll
    for (uint32_t k = 0; k < kCvRun; ++k) {
      const uint64_t t = t0 + min(k, m - 1);
      row[k] = (ntiles >> 32) ? t / a.tiles_per_row : (uint32_t)t / (uint32_t)a.tiles_per_row;
      b0[k] = (t - row[k] * a.tiles_per_row) * kCvTileBytes;
      nv[k] = k < m ? (min(b0[k] + kCvTileBytes, a.row_bytes) - b0[k]) >> 4 : 0;
      const u32x4* src = reinterpret_cast<const u32x4*>(src_s + row[k] * a.row_bytes + b0[k]);
#pragma unroll
      for (int u = 0; u < kCvVecs; ++u) {
        const uint64_t v = (uint64_t)u * kCvThreads + threadIdx.x;
        if (v < nv[k]) x[k][u] = ld16(src + v);
      }
    }
    asm volatile("" ::: "memory");
    uint32_t key[kCvRun], g[kCvRun];
    int32_t tab[kCvRun][PLR_MAX_WORLD];
#pragma unroll
    for (uint32_t k = 0; k < kCvRun; ++k) {
      key[k] = key_of[r0 + (int64_t)row[k]];
      g[k] = seg0 + (uint32_t)(row[k] / kRankSeg);
      if (CPL == 0) {
        const PLR_CONST int32_t* tp = seg_out + g[k] * PLR_MAX_WORLD;
#pragma unroll
        for (int e = 0; e < PLR_MAX_WORLD; ++e) tab[k][e] = tp[e];
      }
    }
    asm volatile("" ::: "memory");
    int64_t out[kCvRun];  // output row of each tile's row; -1: the row is dropped
#pragma unroll
    for (uint32_t k = 0; k < kCvRun; ++k) {
      // branch-free, so that nothing here waits on the loads in flight
      const uint32_t d = key[k] >> 16;  // >= W: not a destination, the row is dropped
      int32_t base;
      if (CPL > 0) {
        int32_t part = 0;
#pragma unroll
        for (int j = 0; j < C; ++j)
          part += ((my_dest[j] < d) | ((my_dest[j] == d) & (my_seg[j] < g[k]))) ? my_cnt[j] : 0;
        base = wave_sum(part);
      } else {
        base = tab[k][0];
#pragma unroll
        for (int e = 1; e < PLR_MAX_WORLD; ++e) base = (d == (uint32_t)e) ? tab[k][e] : base;
      }
      out[k] = d < W ? (int64_t)base + (key[k] & 0xFFFFu) : -1;
    }
#pragma unroll
    for (uint32_t k = 0; k < kCvRun; ++k) {
      if (out[k] < 0) continue;
      u32x4* dst = reinterpret_cast<u32x4*>(a.dst + (uint64_t)out[k] * a.row_bytes + b0[k]);
#pragma unroll
      for (int u = 0; u < kCvVecs; ++u) {
        const uint64_t v = (uint64_t)u * kCvThreads + threadIdx.x;
        if (v < nv[k]) st16(dst + v, x[k][u]);
      }
    }
    // Only calls of more than kCvMaxColumns runs per source take another turn of this loop; the
    // wait keeps its stores from holding registers the next turn's loads and arithmetic
    // reuse (which would put waits for the whole memory queue between them).
    wait_vmem<0>();
  }
}

// The scatter launch of one shape: one workgroup per run of tiles of the longest source
// in grid row s (source s); huge inputs make every row stride over its tiles. The small
// forms have one more column: the workgroup that writes counts and offsets.
template <class Shape>
static void launch_scatter(const CopyVArgs& a, int cpl, hipStream_t s) {
  int64_t most = 0;
  for (uint32_t w = 0; w < a.world; ++w) most = std::max<int64_t>(most, a.row_start[w + 1] - a.row_start[w]);
  const uint32_t gx = cv_grid_columns(cv_tile_columns((uint64_t)most * a.tiles_per_row, Shape::kRun, kCvMaxColumns),
                                      cpl > 0);
  const dim3 b(Shape::kThreads);
  if (cpl == 1)
    launch_dp(k_copy_v_scatter<1, Shape>, dim3(gx, a.world), b, 0, s, false, true, a);
  else if (cpl == 4)
    launch_dp(k_copy_v_scatter<4, Shape>, dim3(gx, a.world), b, 0, s, false, true, a);
  else
    launch_dp(k_copy_v_scatter<0, Shape>, dim3(gx, a.world), b, 0, s, false, true, a);
}

hipError_t launch_copy_v(const CopyVArgs& args, hipStream_t s) {
  CopyVArgs a = args;
  const bool small_rows = a.row_bytes <= kCvSmallRow;
  const uint64_t tile = small_rows ? CvSmall::kTile : CvLarge::kTile;
  a.tiles_per_row = (a.row_bytes + tile - 1) / tile;
  const uint32_t segs = a.seg_start[a.world];
  const uint64_t n = (uint64_t)segs * a.world;
  const int cpl = n <= 64 ? 1 : (n <= kSmallCounts ? 4 : 0);
  a.small = cpl > 0;
  if (a.small) a.xcd = 0;  // the extra column must stay the last workgroup of each row
  launch_dp(k_copy_v_rank, dim3(segs ? segs : 1), dim3(kRankThreads), 0, s, true, false, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (small_rows)
    launch_scatter<CvSmall>(a, cpl, s);
  else
    launch_scatter<CvLarge>(a, cpl, s);
  return hipGetLastError();
}

}  // namespace plr
