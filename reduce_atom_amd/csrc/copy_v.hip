// Variable-length AllToAll packing (MoE dispatch shape).
//
// Purlin paper, appendix C.4 "Variable-Length Collectives" (partition sizes are
// passed at run time) and section 4 (partition offsets come from prefix sums).
// Output rows are packed per destination, in source then row order:
//   kernel 1 (one workgroup per source): counts[s][d] and, for every row, its rank
//            among the earlier rows of the same source bound for the same
//            destination (wave ballots plus a workgroup-wide exclusive scan);
//   kernel 2 (many workgroups): a prologue in every workgroup turns the W*W counts
//            into offsets[d][s] (an exclusive scan in destination-major order),
//            then each wave moves whole rows with 16-byte loads and stores to row
//            offsets[d][s] + rank.
#include "device_common.h"

namespace plr {

constexpr int kRankThreads = 1024;
constexpr int kRankWaves = kRankThreads / 64;

// Kernel 1: one workgroup per source. Rows are taken 1024 at a time in row order,
// one per thread; a wave ballot per destination gives each row its rank among the
// earlier lanes bound for the same destination, per-wave totals in LDS give the
// ranks of earlier waves, and a carry per destination accumulates earlier passes.
__global__ void __launch_bounds__(kRankThreads) k_copy_v_rank(const CopyVArgs a) {
  __shared__ int32_t wave_cnt[kRankWaves][PLR_MAX_WORLD];
  __shared__ int32_t carry[PLR_MAX_WORLD];

  const int s = blockIdx.x;
  const int W = (int)a.world;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int64_t r0 = a.row_start[s];
  const int64_t rows = a.row_start[s + 1] - r0;
  const int32_t* dest = a.dest[s];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes < this one

  if (t < PLR_MAX_WORLD) carry[t] = 0;
  __syncthreads();

  for (int64_t base = 0; base < rows; base += kRankThreads) {
    const int64_t i = base + t;
    const int d = (i < rows) ? dest[i] : -1;
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
      int r = carry[d] + in_wave;
      for (int w2 = 0; w2 < wave; ++w2) r += wave_cnt[w2][d];
      a.rank[r0 + i] = r;
    }
    __syncthreads();  // every thread has read carry and wave_cnt
    if (t < W) {
      int tot = 0;
      for (int w2 = 0; w2 < kRankWaves; ++w2) tot += wave_cnt[w2][t];
      carry[t] += tot;
    }
    __syncthreads();
  }
  if (t < W) a.counts[s * W + t] = carry[t];
}

constexpr int kScatterThreads = 256;
constexpr int kScatterUnroll = 16;

// Kernel 2: a prologue in every workgroup scans the W*W counts (workgroup 0 also
// writes them out as offsets); then wave k of the grid moves row k: all of a
// 14,336-byte row (14 vectors per lane) is in flight at once.
__global__ void __launch_bounds__(kScatterThreads) k_copy_v_scatter(const CopyVArgs a) {
  __shared__ int64_t cnt[PLR_MAX_WORLD * PLR_MAX_WORLD];
  __shared__ int64_t off[PLR_MAX_WORLD * PLR_MAX_WORLD];
  const int W = (int)a.world;
  const int WW = W * W;
  const int t = threadIdx.x;
  if (t < WW) cnt[t] = a.counts[t];
  __syncthreads();
  if (t < WW) {
    // block (d, s): every block of a smaller destination, then the blocks of
    // smaller sources for the same destination
    const int d = t / W, s = t - d * W;
    int64_t o = 0;
    for (int d2 = 0; d2 < d; ++d2)
      for (int s2 = 0; s2 < W; ++s2) o += cnt[s2 * W + d2];
    for (int s2 = 0; s2 < s; ++s2) o += cnt[s2 * W + d];
    off[t] = o;
    if (blockIdx.x == 0) a.offsets[t] = o;
  }
  __syncthreads();

  const int lane = t & 63;
  const uint64_t nvec = a.row_bytes >> 4;
  const int64_t total = a.row_start[W];
  const int waves_per_block = kScatterThreads / 64;
  const int64_t wave = (int64_t)blockIdx.x * waves_per_block + __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * waves_per_block;
  for (int64_t r = wave; r < total; r += nwaves) {
    int s = 0;
    while (r >= a.row_start[s + 1]) ++s;
    const int64_t i = r - a.row_start[s];
    const int32_t d = a.dest[s][i];
    if (d < 0 || d >= W) continue;
    const int64_t out = off[d * W + s] + a.rank[r];
    const u32x4* src = reinterpret_cast<const u32x4*>(a.src[s] + (uint64_t)i * a.row_bytes);
    u32x4* dst = reinterpret_cast<u32x4*>(a.dst + (uint64_t)out * a.row_bytes);
    for (uint64_t v0 = 0; v0 < nvec; v0 += 64 * kScatterUnroll) {
      u32x4 x[kScatterUnroll];
#pragma unroll
      for (int u = 0; u < kScatterUnroll; ++u) {
        const uint64_t v = v0 + (uint64_t)u * 64 + lane;
        if (v < nvec) x[u] = ld16(src + v);
      }
#pragma unroll
      for (int u = 0; u < kScatterUnroll; ++u) {
        const uint64_t v = v0 + (uint64_t)u * 64 + lane;
        if (v < nvec) st16(dst + v, x[u]);
      }
    }
  }
}

hipError_t launch_copy_v(const CopyVArgs& a, uint32_t scatter_grid, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_v_rank, dim3(a.world), dim3(kRankThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_copy_v_scatter, dim3(scatter_grid), dim3(kScatterThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace plr
