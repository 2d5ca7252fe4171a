// Copy kernels: the Atom's copy primitive driven by a compiled layout table.
//
// Purlin paper, section 3.1 "Layouts" (a collective names an input and an output
// layout) and section 3.3 "The Atom" (copy moves bytes between the regions the
// orchestration hands it). Segments of one layout share one length (variable-length
// layouts carry one per segment); each is cut into tiles (one workgroup step) grouped
// into chunks (the notification granule, section 3.2), and a workgroup moves whole
// tiles with 16-byte loads and stores, U vectors in flight per lane. Bytes only:
// nothing passes through a float register path, so every bit pattern is preserved.
#include "device_common.h"

namespace plr {

template <int U>
__global__ void __launch_bounds__(512) k_copy_direct(const CopyArgs a) {
  const uint32_t nthr = blockDim.x;
  uint32_t ready = 0xFFFFFFFFu;  // flag (source, chunk) this workgroup has already seen
  const bool wait = must_wait(a.nt);
  const uint32_t b = logical_block(a.xcd);
  const uint32_t t_end = min(a.ntiles, (b + 1) * a.run);
  for (uint32_t t = b * a.run; t < t_end; ++t) {
    uint32_t seg, part, c, c_last;
    uint64_t len, b0, b1;  // the tile: bytes [b0, b1) of its segment
    if (a.mode == kCopyVar) {
      // the last segment starting at or before t owns it (empty segments share the
      // first tile of the next one; entries past the last segment hold ~0u)
      seg = 0;
#pragma unroll
      for (uint32_t k = 1; k < PLR_MAX_WORLD; ++k) seg = t >= a.var_tile0[k] ? k : seg;
      part = t - a.var_tile0[seg];
      len = a.var_len[seg];
      const uint64_t sh = a.var_shift[seg];
      b0 = part ? (uint64_t)part * a.tile_bytes - sh : 0;
      b1 = min((uint64_t)(part + 1) * a.tile_bytes - sh, len);
      const uint64_t cb = (uint64_t)a.tiles_per_chunk * a.tile_bytes;
      c = a.var_chunk0[seg] + (uint32_t)(b0 / cb);
      c_last = a.var_chunk0[seg] + (uint32_t)((b1 - 1) / cb);
    } else {
      seg = t / a.tiles_per_seg;
      part = t - seg * a.tiles_per_seg;
      len = a.seg_len;
      b0 = (uint64_t)part * a.tile_bytes;
      b1 = min(b0 + a.tile_bytes, len);
      c = c_last = seg * a.chunks_per_seg + part / a.tiles_per_chunk;
    }
    uint32_t s;
    uint64_t src_off, dst_off;
    if (a.mode != kCopyTransposed) {
      s = a.seg_src[seg];
      src_off = a.seg_src_off[seg];
      dst_off = a.seg_dst_off[seg];
    } else {  // transposed: segment k = s*W + d
      s = seg / a.world;
      const uint32_t d = seg - s * a.world;
      src_off = (uint64_t)d * a.slice;
      dst_off = ((uint64_t)d * a.world + s) * a.slice;
    }
    if (wait) {  // flags follow the segments, source by source
      for (uint32_t f = c; f <= c_last; ++f) {
        if (f != ready) {
          if (!wg_wait_flags(a.nt, f, 0, 1)) return;
          ready = f;
        }
      }
    }
    const uint64_t nv = (b1 - b0) >> 4;
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

// Segment addressing of tile t: source index, source and destination byte offsets.
__device__ __forceinline__ void copy_tile_addr(const CopyArgs& a, uint32_t t, uint32_t& seg,
                                               uint32_t& part, uint32_t& s, uint64_t& src_off,
                                               uint64_t& dst_off) {
  seg = t / a.tiles_per_seg;
  part = t - seg * a.tiles_per_seg;
  if (a.mode == kCopyTable) {
    s = a.seg_src[seg];
    src_off = a.seg_src_off[seg];
    dst_off = a.seg_dst_off[seg];
  } else {
    s = seg / a.world;
    const uint32_t d = seg - s * a.world;
    src_off = (uint64_t)d * a.slice;
    dst_off = ((uint64_t)d * a.world + s) * a.slice;
  }
}

// LDS-staged variant (PLR_PATH_LDS): a workgroup of 256 threads walks its run of
// tiles as 4 KiB slabs (1 KiB per wave); each wave keeps kCopyStages slabs in flight
// through a private LDS ring (global->LDS DMA), waits only for the oldest, reads it
// back and stores it at the layout's destination. Chunk flags are awaited before the
// first DMA of a chunk.

__global__ void __launch_bounds__(256) k_copy_lds(const CopyArgs a) {
  __shared__ u32x4 ring[4][kCopyStages][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t spt = (uint32_t)((a.tile_bytes + 4095) / 4096);  // slabs per tile
  const uint32_t t0 = logical_block(a.xcd) * a.run;
  const uint32_t t1 = min(a.ntiles, t0 + a.run);
  const uint32_t j1 = (t1 - t0) * spt;
  uint32_t ready = 0xFFFFFFFFu;
  const bool wait = must_wait(a.nt);

  // byte offset of this lane's vector inside slab j's segment, and whether it exists
  auto where = [&](uint32_t j, uint32_t& s, uint64_t& src_b, uint64_t& dst_b, bool& valid) -> uint32_t {
    const uint32_t t = t0 + j / spt;
    uint32_t seg, part;
    uint64_t so, dof;
    copy_tile_addr(a, t, seg, part, s, so, dof);
    const uint64_t b = (uint64_t)part * a.tile_bytes + (j % spt) * 4096 + (uint64_t)wave * 1024;
    const uint64_t tile_end = min((uint64_t)(part + 1) * a.tile_bytes, a.seg_len);
    const uint64_t bl = b + (uint64_t)lane * 16;
    valid = bl < tile_end;
    const uint64_t bc = valid ? bl : a.seg_len - 16;  // ragged lanes re-read a valid vector
    src_b = so + bc;
    dst_b = dof + bl;
    return seg * a.chunks_per_seg + part / a.tiles_per_chunk;
  };

  auto stage = [&](uint32_t j) -> bool {
    uint32_t s;
    uint64_t src_b, dst_b;
    bool valid;
    const uint32_t c = where(j, s, src_b, dst_b, valid);
    if (wait) {
      const uint32_t f = c;  // flags follow the segments, source by source
      if (f != ready) {
        if (!wg_wait_flags(a.nt, f, 0, 1)) return false;
        ready = f;
      }
    }
    lds_dma16(a.src[s] + src_b, (PLR_LDS void*)&ring[wave][j % kCopyStages][0]);
    return true;
  };

  for (uint32_t k = 0; k < kCopyStages - 1; ++k)
    if (k < j1 && !stage(k)) {
      wait_vmem<0>();
      return;
    }
  for (uint32_t j = 0; j < j1; ++j) {
    if (j + kCopyStages - 1 < j1) {
      if (!stage(j + kCopyStages - 1)) {
        wait_vmem<0>();
        return;
      }
      wait_vmem<kCopyStages - 1>();
    } else {
      // the last slabs: this also waits for the previous slab's store, which measured
      // faster than waiting for the DMAs alone and storing the last slabs together
      // (8 x 64 MiB AllGather 170.6-172.5 against 179.6-181.4 us)
      wait_vmem<0>();
    }
    u32x4 x[1];
    lds_read_wait<1>((const PLR_LDS u32x4*)&ring[wave][j % kCopyStages][lane], x);
    uint32_t s;
    uint64_t src_b, dst_b;
    bool valid;
    where(j, s, src_b, dst_b, valid);
    if (valid) st16(reinterpret_cast<u32x4*>(a.dst + dst_b), x[0]);
  }
}

hipError_t launch_copy(const CopyArgs& a, const Launch& l, hipStream_t s) {
  dim3 g(l.grid), b(l.block);
  if (l.datapath == PLR_PATH_LDS) {
    if (l.block != 256) return hipErrorInvalidValue;
    launch_dp(k_copy_lds, g, b, 0, s, true, true, a);
    return hipGetLastError();
  }
  switch (l.unroll) {
    case 1: launch_dp(k_copy_direct<1>, g, b, l.lds_bytes, s, true, true, a); break;
    case 2: launch_dp(k_copy_direct<2>, g, b, l.lds_bytes, s, true, true, a); break;
    case 4: launch_dp(k_copy_direct<4>, g, b, l.lds_bytes, s, true, true, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace plr
