// Copy kernels: the Atom's copy primitive driven by a compiled layout table.
//
// Purlin paper, section 3.1 "Layouts" (a collective names an input and an output
// layout) and section 3.3 "The Atom" (copy moves bytes between the regions the
// orchestration hands it). Segments of one layout share one length; each is cut
// into tiles (one workgroup step) grouped into chunks (the notification granule,
// section 3.2), and a workgroup moves whole tiles with 16-byte loads and stores,
// U vectors in flight per lane. Bytes only:
// nothing passes through a float register path, so every bit pattern is preserved.
#include "device_common.h"

namespace plr {

template <int U>
__global__ void __launch_bounds__(512) k_copy_direct(const CopyArgs a) {
  const uint32_t nthr = blockDim.x;
  uint32_t ready = 0xFFFFFFFFu;  // flag (source, chunk) this workgroup has already seen
  const uint32_t t_end = min(a.ntiles, (blockIdx.x + 1) * a.run);
  for (uint32_t t = blockIdx.x * a.run; t < t_end; ++t) {
    const uint32_t seg = t / a.tiles_per_seg;
    const uint32_t part = t - seg * a.tiles_per_seg;
    uint32_t s;
    uint64_t src_off, dst_off;
    if (a.mode == kCopyTable) {
      s = a.seg_src[seg];
      src_off = a.seg_src_off[seg];
      dst_off = a.seg_dst_off[seg];
    } else {  // transposed: segment k = s*W + d
      s = seg / a.world;
      const uint32_t d = seg - s * a.world;
      src_off = (uint64_t)d * a.slice;
      dst_off = ((uint64_t)d * a.world + s) * a.slice;
    }
    if (a.nt.flags) {
      const uint32_t c = seg * a.chunks_per_seg + part / a.tiles_per_chunk;
      const uint32_t f = s * a.nchunks + c;
      if (f != ready) {
        if (!wg_wait_flags(a.nt, a.nt.flags + f, 0, 1)) return;
        ready = f;
      }
    }
    const uint64_t b0 = (uint64_t)part * a.tile_bytes;
    const uint64_t nv = (min(b0 + a.tile_bytes, a.seg_len) - b0) >> 4;
    const u32x4* src = reinterpret_cast<const u32x4*>(a.src[s] + src_off + b0);
    u32x4* dst = reinterpret_cast<u32x4*>(a.dst + dst_off + b0);
    uint64_t v = threadIdx.x;
    for (; v + (uint64_t)(U - 1) * nthr < nv; v += (uint64_t)U * nthr) {
      u32x4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = ld16(src + v + (uint64_t)u * nthr);
#pragma unroll
      for (int u = 0; u < U; ++u) st16(dst + v + (uint64_t)u * nthr, x[u]);
    }
    for (; v < nv; v += nthr) st16(dst + v, ld16(src + v));
  }
}

hipError_t launch_copy(const CopyArgs& a, const Launch& l, hipStream_t s) {
  dim3 g(l.grid), b(l.block);
  switch (l.unroll) {
    case 1: hipLaunchKernelGGL((k_copy_direct<1>), g, b, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_copy_direct<2>), g, b, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_copy_direct<4>), g, b, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace plr
