// AllReduce of W contributions into W outputs on one GPU (every output is the
// source-order fp32 reduction of all W contributions).
//
// Purlin paper, section 3.1 "Layouts": AllReduce is ReduceScatter followed by
// AllGather, a scattered-to-scattered transformation, and compatible transforms are
// composed into one kernel; section 3.2 "SNAC": for the composed AllReduce, staging,
// reduction and gathering roles work on chunks so that they overlap, and a chunk is
// consumed only after its producer's notification.
//
// Two datapaths:
//  - fused (PLR_PATH_DIRECT): one workgroup reduces a tile and stores the result to
//    all W outputs. With every contribution in one GPU's memory this moves the fewest
//    bytes (W reads + W writes per output element).
//  - composed (PLR_PATH_COMPOSED): the SNAC role split inside one kernel. Workgroup b
//    first acts as a reducer for tile b: it reduces the tile into the output of the
//    rank that owns the tile's slice, then releases the tile's flag (agent scope).
//    It then acts as a gatherer for tile b - lag: it waits for that tile's flag,
//    acquires, and copies the reduced tile into the other W-1 outputs. A workgroup
//    only ever waits for a lower-numbered workgroup, whose reduction never waits;
//    workgroups go round-robin to the 8 XCDs and each XCD dispatches its own in
//    increasing order, and lag is a multiple of 8, so the producer is on the same XCD
//    and was dispatched first: the waits always end. A bounded spin turns any
//    surprise into PLR_ETIMEOUT.
#include "device_common.h"

namespace plr {

// tile t -> first vector and vector count inside the share; tiles never cross slices
__device__ __forceinline__ void ar_tile(const AllReduceArgs& a, uint32_t t, uint32_t& owner,
                                        uint64_t& v0, uint64_t& nv) {
  owner = t / a.tiles_per_slice;
  const uint32_t part = t - owner * a.tiles_per_slice;
  const uint64_t off = (uint64_t)part * a.tile_vecs;
  v0 = (uint64_t)owner * a.slice_vecs + off;
  nv = min(a.tile_vecs, a.slice_vecs - off);
}

template <int DT, int W>
__global__ void __launch_bounds__(512) k_allreduce_fused(const AllReduceArgs a) {
  const uint32_t t_end = min(a.ntiles, (blockIdx.x + 1) * a.run);
  for (uint32_t t = blockIdx.x * a.run; t < t_end; ++t) {
    uint32_t owner;
    uint64_t v0, nv;
    ar_tile(a, t, owner, v0, nv);
    for (uint64_t k = threadIdx.x; k < nv; k += blockDim.x) {
      u32x4 x[W];
#pragma unroll
      for (int w = 0; w < W; ++w) x[w] = ld16(a.src[w] + v0 + k);
      const u32x4 y = combine<DT, W>(x);
#pragma unroll
      for (int w = 0; w < W; ++w) st16(a.dst[w] + v0 + k, y);
    }
  }
}

template <int DT, int W>
__global__ void __launch_bounds__(512) k_allreduce_composed(const AllReduceArgs a) {
  const uint32_t b = blockIdx.x;
  // reducer role: tile b into its owner's output, then release the tile's flag
  if (b < a.ntiles) {
    uint32_t owner;
    uint64_t v0, nv;
    ar_tile(a, b, owner, v0, nv);
    // A plain store, not a non-temporal one: the gatherer re-reads this tile shortly
    // after, and with plain stores the kernel runs 7% faster (the re-read leaves the
    // L2 either way: the L2's fetch counters read the same).
    for (uint64_t k = threadIdx.x; k < nv; k += blockDim.x) {
      u32x4 x[W];
#pragma unroll
      for (int w = 0; w < W; ++w) x[w] = ld16(a.src[w] + v0 + k);
      a.dst[owner][v0 + k] = combine<DT, W>(x);
    }
    __syncthreads();  // every wave's stores precede the release below
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_store(const_cast<uint64_t*>(a.nt.flags) + b, a.nt.epoch, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // gatherer role: tile b - lag, produced by a lower-numbered workgroup
  if (b < a.lag) return;
  const uint32_t g = b - a.lag;
  if (g >= a.ntiles) return;
  if (!wg_wait_flags(a.nt, g, 0, 1)) return;
  uint32_t owner;
  uint64_t v0, nv;
  ar_tile(a, g, owner, v0, nv);
  for (uint64_t k = threadIdx.x; k < nv; k += blockDim.x) {
    const u32x4 y = ld16(a.dst[owner] + v0 + k);
#pragma unroll
    for (int w = 0; w < W; ++w)
      if (w != (int)owner) st16(a.dst[w] + v0 + k, y);
  }
}

template <int DT, int W>
static hipError_t launch_ar_w(const AllReduceArgs& a, const Launch& l, hipStream_t s) {
  dim3 g(l.grid), bl(l.block);
  if (l.datapath == PLR_PATH_COMPOSED)
    launch_dp(k_allreduce_composed<DT, W>, g, bl, 0, s, true, true, a);
  else
    launch_dp(k_allreduce_fused<DT, W>, g, bl, l.lds_bytes, s, true, true, a);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_ar_dt(const AllReduceArgs& a, const Launch& l, hipStream_t s) {
  switch (a.world) {
#define PLR_W(w) \
  case w: return launch_ar_w<DT, w>(a, l, s);
    PLR_W(1) PLR_W(2) PLR_W(3) PLR_W(4) PLR_W(5) PLR_W(6) PLR_W(7) PLR_W(8)
    PLR_W(9) PLR_W(10) PLR_W(11) PLR_W(12) PLR_W(13) PLR_W(14) PLR_W(15) PLR_W(16)
#undef PLR_W
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_allreduce(const AllReduceArgs& a, int dtype, const Launch& l, hipStream_t s) {
  switch (dtype) {
    case PLR_BF16: return launch_ar_dt<PLR_BF16>(a, l, s);
    case PLR_F16: return launch_ar_dt<PLR_F16>(a, l, s);
    case PLR_F32: return launch_ar_dt<PLR_F32>(a, l, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace plr
