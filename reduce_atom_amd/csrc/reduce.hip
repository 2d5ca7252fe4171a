// Reduce kernels: the Atom's ordered (SCORE) reduction of W sources into one share.
//
// Purlin paper, section 3.3 "The Atom": every output element is owned by one thread,
// which accumulates the sources in a fixed order; source fetches are pipelined and
// several independent accumulators are kept in flight. Here a lane owns one 16-byte
// output vector per pipeline step (8 bf16/fp16 or 4 fp32 elements, each with its own
// binary32 accumulator) and `U` such vectors per step, so W*U 16-byte loads are in
// flight per lane before the first add.
//
// Work division: the share is cut into tiles of `tile_vecs` vectors, the step one
// workgroup consumes; tiles_per_chunk consecutive tiles form a chunk, the
// notification granule (section 3.2). Workgroup b consumes the run of tiles
// [b*run, (b+1)*run); when the call is notified, the workgroup waits for a chunk's W
// flags before its first tile of that chunk.
#include "device_common.h"

namespace plr {

template <int DT, int W, int U>
__global__ void __launch_bounds__(512) k_reduce_direct(const ReduceArgs a) {
  const uint32_t nthr = blockDim.x;
  uint32_t ready = 0xFFFFFFFFu;  // chunk whose flags this workgroup has already seen
  const bool wait = must_wait(a.nt);
  const uint32_t b = logical_block(a.xcd);
  const uint32_t t_end = min(a.ntiles, (b + 1) * a.run);
  for (uint32_t t = b * a.run; t < t_end; ++t) {
    if (wait) {
      const uint32_t c = t / a.tiles_per_chunk;
      if (c != ready) {
        if (!wg_wait_flags(a.nt, c, a.nchunks, W)) return;
        ready = c;
      }
    }
    const uint64_t v_end = min((uint64_t)(t + 1) * a.tile_vecs, a.nvec);
    uint64_t v = (uint64_t)t * a.tile_vecs + threadIdx.x;
    // full pipeline steps: U vectors per lane, all W*U loads issued before any add
    for (; v + (uint64_t)(U - 1) * nthr < v_end; v += (uint64_t)U * nthr) {
      u32x4 x[U][W];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int w = 0; w < W; ++w) x[u][w] = ld16(a.src[w] + v + (uint64_t)u * nthr);
#pragma unroll
      for (int u = 0; u < U; ++u) st16(a.dst + v + (uint64_t)u * nthr, combine<DT, W>(x[u]));
    }
    // ragged end of the tile: one vector at a time
    for (; v < v_end; v += nthr) {
      u32x4 x[W];
#pragma unroll
      for (int w = 0; w < W; ++w) x[w] = ld16(a.src[w] + v);
      st16(a.dst + v, combine<DT, W>(x));
    }
  }
}

// LDS-staged variant (PLR_PATH_LDS): the SNAC stage / consume split made explicit.
// A workgroup of 256 threads walks its run of tiles as slabs of 256 vectors per
// source; wave k owns vectors [64k, 64k+64) of every slab and a private ring of S
// stages in LDS (S x W x 1 KiB per wave). The wave issues the DMA of slab j+S-1 into
// its ring, waits only for slab j, reads slab j's W vectors back from LDS, reduces
// them in source order and stores. Chunk flags are awaited (by the whole workgroup)
// before the first DMA into a new chunk.
template <int W>
struct LdsRing {
  static constexpr int S = lds_reduce_stages(W);  // S*W*4 KiB <= 128 KiB
};

template <int DT, int W>
__global__ void __launch_bounds__(256) k_reduce_lds(const ReduceArgs a) {
  constexpr int S = LdsRing<W>::S;
  __shared__ u32x4 ring[4][S][W][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // tiles are whole slabs (or the share is a single tile shorter than one slab)
  const uint64_t slabs_per_tile = (a.tile_vecs + 255) / 256;
  const uint64_t nslab_all = (a.nvec + 255) / 256;
  const uint32_t b = logical_block(a.xcd);
  const uint64_t j0 = (uint64_t)b * a.run * slabs_per_tile;
  const uint64_t j1 = min(nslab_all, (uint64_t)(b + 1) * a.run * slabs_per_tile);
  uint32_t ready = 0xFFFFFFFFu;
  const bool wait = must_wait(a.nt);

  // stage slab j: every wave always issues exactly W DMAs (ragged lanes re-read the
  // last vector instead of skipping), so the wait counts stay exact
  auto stage = [&](uint64_t j) -> bool {
    if (wait) {
      const uint32_t c = (uint32_t)(j / slabs_per_tile) / a.tiles_per_chunk;
      if (c != ready) {
        if (!wg_wait_flags(a.nt, c, a.nchunks, W)) return false;
        ready = c;
      }
    }
    const uint64_t v = min(j * 256 + (uint64_t)wave * 64 + lane, a.nvec - 1);
    const int st = (int)(j % S);
#pragma unroll
    for (int w = 0; w < W; ++w) lds_dma16(a.src[w] + v, (PLR_LDS void*)&ring[wave][st][w][0]);
    return true;
  };

  for (int k = 0; k < S - 1; ++k)
    if (j0 + k < j1 && !stage(j0 + k)) {
      wait_vmem<0>();
      return;
    }
  for (uint64_t j = j0; j < j1; ++j) {
    if (j + S - 1 < j1) {
      if (!stage(j + S - 1)) {
        wait_vmem<0>();
        return;
      }
      wait_vmem<(S - 1) * W>();
    } else {
      wait_vmem<0>();
    }
    const int st = (int)(j % S);
    u32x4 x[W];  // ring[wave][st][w][lane] sits 1 KiB after ring[wave][st][w - 1][lane]
    lds_read_wait<W>((const PLR_LDS u32x4*)&ring[wave][st][0][lane], x);
    const uint64_t v = j * 256 + (uint64_t)wave * 64 + lane;
    if (v < a.nvec) st16(a.dst + v, combine<DT, W>(x));
  }
}

template <int DT, int W>
static hipError_t launch_w(const ReduceArgs& a, const Launch& l, hipStream_t s) {
  dim3 g(l.grid), b(l.block);
  if (l.datapath == PLR_PATH_LDS) {
    if (l.block != 256) return hipErrorInvalidValue;
    launch_dp(k_reduce_lds<DT, W>, g, b, 0, s, true, true, a);
    return hipGetLastError();
  }
  switch (l.unroll) {
    case 1: launch_dp(k_reduce_direct<DT, W, 1>, g, b, l.lds_bytes, s, true, true, a); break;
    case 2: launch_dp(k_reduce_direct<DT, W, 2>, g, b, l.lds_bytes, s, true, true, a); break;
    case 4: launch_dp(k_reduce_direct<DT, W, 4>, g, b, l.lds_bytes, s, true, true, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_dt(const ReduceArgs& a, const Launch& l, hipStream_t s) {
  switch (a.world) {
#define PLR_W(w) \
  case w: return launch_w<DT, w>(a, l, s);
    PLR_W(1) PLR_W(2) PLR_W(3) PLR_W(4) PLR_W(5) PLR_W(6) PLR_W(7) PLR_W(8)
    PLR_W(9) PLR_W(10) PLR_W(11) PLR_W(12) PLR_W(13) PLR_W(14) PLR_W(15) PLR_W(16)
#undef PLR_W
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_reduce(const ReduceArgs& a, int dtype, const Launch& l, hipStream_t s) {
  switch (dtype) {
    case PLR_BF16: return launch_dt<PLR_BF16>(a, l, s);
    case PLR_F16: return launch_dt<PLR_F16>(a, l, s);
    case PLR_F32: return launch_dt<PLR_F32>(a, l, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace plr
