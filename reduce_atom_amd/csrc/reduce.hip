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
  const uint32_t t_end = min(a.ntiles, (blockIdx.x + 1) * a.run);
  for (uint32_t t = blockIdx.x * a.run; t < t_end; ++t) {
    if (a.nt.flags) {
      const uint32_t c = t / a.tiles_per_chunk;
      if (c != ready) {
        if (!wg_wait_flags(a.nt, a.nt.flags + c, a.nchunks, W)) return;
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

template <int DT, int W>
static hipError_t launch_w(const ReduceArgs& a, const Launch& l, hipStream_t s) {
  dim3 g(l.grid), b(l.block);
  switch (l.unroll) {
    case 1: hipLaunchKernelGGL((k_reduce_direct<DT, W, 1>), g, b, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_reduce_direct<DT, W, 2>), g, b, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_reduce_direct<DT, W, 4>), g, b, 0, s, a); break;
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
