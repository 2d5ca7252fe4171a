// Variable-length AllToAll packing (MoE dispatch shape).
//
// Purlin paper, appendix C.4 "Variable-Length Collectives" (partition sizes are
// passed at run time) and section 4 (partition offsets come from prefix sums).
// Output rows are packed per destination, in source then row order:
//   kernel 1 (one workgroup per 1024-row segment of a source): for every row, its
//            rank among the earlier rows of its segment bound for the same
//            destination (wave ballots plus a workgroup-wide exclusive scan), and the
//            segment's counts; the last of those workgroups scans the segments into
//            per-segment bases, counts[s][d] and offsets[d][s] (an exclusive scan in
//            destination-major order);
//   kernel 2 (one wave per row): moves whole rows with 16-byte loads and stores to
//            row offsets[d][s] + rank.
#include "device_common.h"

namespace plr {

constexpr int kRankThreads = kRankSeg;
constexpr int kRankWaves = kRankThreads / 64;

// Kernel 1: one workgroup per segment of kRankSeg consecutive rows of one source, one
// row per thread. A wave ballot per destination gives each row its rank among the
// lower lanes bound for the same destination, and per-wave totals in LDS the rank
// across waves: the row's rank inside its segment. The segment's per-destination
// counts go to scratch. The last workgroup to finish (a ticket counter in scratch,
// acquire-release at agent scope, left at zero again) scans them: per source and
// destination the rows of earlier segments (seg_base), the totals counts[s][d], and
// offsets[d][s] (an exclusive scan in destination-major order).
__global__ void __launch_bounds__(kRankThreads) k_copy_v_rank(const CopyVArgs a) {
  __shared__ int32_t wave_cnt[kRankWaves][PLR_MAX_WORLD];
  __shared__ int64_t tot[PLR_MAX_WORLD * PLR_MAX_WORLD];
  __shared__ int last;

  const int W = (int)a.world;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const uint32_t seg = blockIdx.x;
  int s = 0;
  while (seg >= a.seg_start[s + 1]) ++s;
  const int64_t i = (int64_t)(seg - a.seg_start[s]) * kRankSeg + t;  // row within source s
  const int64_t rows = a.row_start[s + 1] - a.row_start[s];
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
  if (d >= 0 && d < W) {
    int r = in_wave;
    for (int w2 = 0; w2 < wave; ++w2) r += wave_cnt[w2][d];
    a.rank[a.row_start[s] + i] = r;
  }
  if (t < W) {
    int c = 0;
    for (int w2 = 0; w2 < kRankWaves; ++w2) c += wave_cnt[w2][t];
    a.seg_count[(uint64_t)seg * W + t] = c;
  }

  // ticket: the last workgroup sees every segment's counts
  __syncthreads();
  if (t == 0) {
    const uint32_t done = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = (done == gridDim.x - 1);
  }
  __syncthreads();
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int WW = W * W;
  if (t < WW) {  // thread (s2, d2): scan source s2's segments for destination d2
    const int s2 = t / W, d2 = t - s2 * W;
    int64_t run = 0;
    for (uint32_t g = a.seg_start[s2]; g < a.seg_start[s2 + 1]; ++g) {
      a.seg_base[(uint64_t)g * W + d2] = (int32_t)run;
      run += __hip_atomic_load(a.seg_count + (uint64_t)g * W + d2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    tot[t] = run;  // counts[s2][d2]
    a.counts[t] = run;
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
    a.offsets[t] = o;
  }
  if (t == 0) __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kScatterThreads = 256;
constexpr int kScatterUnroll = 16;

// Kernel 2: wave k of the grid moves row k. The row's loads are issued first (a
// source row exists whatever its destination); its destination, rank and block
// offset are read meanwhile, and the stores go to row offsets[d][s] + rank. All of a
// 14,336-byte row (14 vectors per lane) is in flight at once.
__global__ void __launch_bounds__(kScatterThreads) k_copy_v_scatter(const CopyVArgs a) {
  const int W = (int)a.world;
  const int lane = threadIdx.x & 63;
  const uint64_t nvec = a.row_bytes >> 4;
  const int64_t total = a.row_start[W];
  const int waves_per_block = kScatterThreads / 64;
  const int64_t wave =
      (int64_t)logical_block(a.xcd) * waves_per_block + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * waves_per_block;
  for (int64_t r = wave; r < total; r += nwaves) {
    int s = 0;
    while (r >= a.row_start[s + 1]) ++s;
    const int64_t i = r - a.row_start[s];
    const u32x4* src = reinterpret_cast<const u32x4*>(a.src[s] + (uint64_t)i * a.row_bytes);
    for (uint64_t v0 = 0; v0 < nvec; v0 += 64 * kScatterUnroll) {
      u32x4 x[kScatterUnroll];
#pragma unroll
      for (int u = 0; u < kScatterUnroll; ++u) {
        const uint64_t v = v0 + (uint64_t)u * 64 + lane;
        if (v < nvec) x[u] = ld16(src + v);
      }
      const int32_t d = a.dest[s][i];
      if (d < 0 || d >= W) break;  // not a destination: the row is dropped
      const uint64_t g = a.seg_start[s] + (uint64_t)(i / kRankSeg);
      const int64_t out = a.offsets[d * W + s] + a.seg_base[g * W + d] + a.rank[r];
      u32x4* dst = reinterpret_cast<u32x4*>(a.dst + (uint64_t)out * a.row_bytes);
#pragma unroll
      for (int u = 0; u < kScatterUnroll; ++u) {
        const uint64_t v = v0 + (uint64_t)u * 64 + lane;
        if (v < nvec) st16(dst + v, x[u]);
      }
    }
  }
}

hipError_t launch_copy_v(const CopyVArgs& a, uint32_t scatter_grid, hipStream_t s) {
  const uint32_t segs = a.seg_start[a.world];
  hipLaunchKernelGGL(k_copy_v_rank, dim3(segs ? segs : 1), dim3(kRankThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_copy_v_scatter, dim3(scatter_grid), dim3(kScatterThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace plr
