/*
 * plr_atom.h - device-callable Atom for gfx950 (AMD Instinct MI355X), HIP only.
 *
 * The Atom is the datapath layer of Purlin (Aimuyo, Gandhi, Kozyrakis, "Purlin:
 * Separating Orchestration from the Datapath of Collectives", section 3.3 "The Atom"):
 * the copy and the reduce primitives. The project README ("Device-side") lets a user
 * kernel call them itself, one workgroup of the Atom's THREADS threads per slice, with
 * the Atom's workspace bytes of workgroup-local memory, so that collective data
 * movement fuses with the user's own work (section 2.1: device-side primitives that
 * applications can schedule and compose). The library's own kernels are built from the
 * same functions.
 *
 * Contract of every function here:
 *   - it is called by all THREADS threads of one workgroup together (blockDim.x ==
 *     THREADS), like a workgroup barrier; it contains none itself;
 *   - device addresses and byte counts are multiples of 16 (one 16-byte vector per
 *     lane per step), and a destination does not overlap its sources;
 *   - loads and stores are 16 bytes wide and non-temporal (every byte is touched once);
 *   - the reduction is the Atom's ordered one (SCORE, section 3.3): each output element
 *     is owned by one lane, which widens source 0 exactly, adds sources 1..W-1 in order
 *     in binary32, and rounds once to nearest-even into the element type, so results are
 *     bitwise repeatable and independent of THREADS and UNROLL;
 *   - the direct datapath stages through registers, so COPY_LDS_BYTES and
 *     REDUCE_LDS_BYTES are 0 and the workspace argument of the pages' interface is not
 *     needed.
 *
 * Notification (section 3.2 "SNAC"): signal_flag publishes a chunk (release at agent
 * scope, after every store the calling workgroup made), wait_flag consumes it (acquire
 * at agent scope: the workgroup's later loads see the producer's stores). Flags hold
 * a monotonic epoch (section 4.3 "Epoch Bookkeeping"), and a wait accepts any value at
 * or above its epoch, so a chunk's buffer must not be rewritten (or signalled for a later
 * epoch) before its consumer has finished reading it. A wait is bounded: it returns
 * false after spin_limit polls, and a kernel must then give up without reading.
 * Packets (section 3.2 and Figure 7: payload and notification in one store): a producer
 * may write its share directly in the packet form plr_reduce_packets reads
 * (packet_slot, store_packet), so that it needs neither a flag nor a release.
 *
 * Policy (section 4.2 "Codesign Policies and Tuning": applications may define their
 * own): THREADS (64, 128, 256 or 512) and UNROLL (16-byte vectors per lane in flight
 * per source, 1, 2 or 4; a reduce holds UNROLL x W vectors per lane, and beyond about 56
 * of them, e.g. UNROLL 4 with W >= 15, the compiler spills registers). The library's measured gfx950 choice for streaming shares is
 * 128 threads, 1 vector, one 2 KiB slice per workgroup and a grid that covers the data.
 */
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "plr.h"

namespace plr {
namespace atom {

typedef uint32_t vec16 __attribute__((ext_vector_type(4)));  // one 16-byte vector

// ---- 16-byte streaming access ----
__device__ __forceinline__ vec16 load16(const vec16* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store16(vec16* p, vec16 v) { __builtin_nontemporal_store(v, p); }

// ---- element types inside one 16-byte vector ----
// Element j of a vector is at bits [16j, 16j+16) of the little-endian 128-bit word
// (32j for fp32). Widening is exact; narrowing is one round-to-nearest-even.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int DT>
struct Elems;

template <>
struct Elems<PLR_BF16> {
  static constexpr int N = 8;
  __device__ static __forceinline__ void widen(vec16 v, float* f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = __uint_as_float(v[k] << 16);
      f[2 * k + 1] = __uint_as_float(v[k] & 0xFFFF0000u);
    }
  }
  __device__ static __forceinline__ vec16 narrow(const float* f) {
    vec16 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bf16x2 b = __builtin_convertvector((f32x2){f[2 * k], f[2 * k + 1]}, bf16x2);
      r[k] = __builtin_bit_cast(uint32_t, b);
    }
    return r;
  }
};

template <>
struct Elems<PLR_F16> {
  static constexpr int N = 8;
  // Scalar conversions with explicit bit packing: v_cvt_f32_f16 widens exactly and
  // v_cvt_f16_f32 rounds to nearest even (denormals kept, the kernels' float mode).
  __device__ static __forceinline__ void widen(vec16 v, float* f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[k] & 0xFFFFu));
      f[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[k] >> 16));
    }
  }
  __device__ static __forceinline__ vec16 narrow(const float* f) {
    vec16 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)f[2 * k]);
      const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)f[2 * k + 1]);
      r[k] = lo | (hi << 16);
    }
    return r;
  }
};

template <>
struct Elems<PLR_F32> {
  static constexpr int N = 4;
  __device__ static __forceinline__ void widen(vec16 v, float* f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(v[k]);
  }
  __device__ static __forceinline__ vec16 narrow(const float* f) {
    vec16 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = __float_as_uint(f[k]);
    return r;
  }
};

// Epilogues run on the binary32 accumulators of one 16-byte output vector, before the
// single rounding. An epilogue type provides
//   Pre  load(uint64_t vec) const   issued together with the sources' loads of output
//                                   vector `vec` (so that its own loads overlap them);
//   void operator()(float* acc, int n, uint64_t first_element, const Pre&) const
//                                   transforms the n accumulators in place.
// No epilogue: the accumulators are rounded as they are.
struct NoEpilogue {
  struct Pre {};
  __device__ __forceinline__ Pre load(uint64_t) const { return {}; }
  __device__ __forceinline__ void operator()(float*, int, uint64_t, const Pre&) const {}
};

// SCORE combine of one vector per source (x[0..W-1], in source order): binary32
// accumulation from source 0, then the epilogue, then one round-to-nearest-even.
template <int DT, int W, class Epi = NoEpilogue>
__device__ __forceinline__ vec16 combine(const vec16* x, uint64_t first_element = 0, const Epi& epi = Epi(),
                                         const typename Epi::Pre& pre = typename Epi::Pre()) {
  constexpr int N = Elems<DT>::N;
  float acc[N];
  Elems<DT>::widen(x[0], acc);
#pragma unroll
  for (int w = 1; w < W; ++w) {
    float t[N];
    Elems<DT>::widen(x[w], t);
#pragma unroll
    for (int j = 0; j < N; ++j) acc[j] = acc[j] + t[j];
  }
  epi(acc, N, first_element, pre);
  return Elems<DT>::narrow(acc);
}

// ---- the Atom ----
template <int THREADS_ = 128, int UNROLL_ = 1>
struct Atom {
  static constexpr int THREADS = THREADS_;
  static constexpr int UNROLL = UNROLL_;
  static constexpr size_t COPY_LDS_BYTES = 0;
  static constexpr size_t REDUCE_LDS_BYTES = 0;
  static_assert(THREADS == 64 || THREADS == 128 || THREADS == 256 || THREADS == 512, "THREADS");
  static_assert(UNROLL == 1 || UNROLL == 2 || UNROLL == 4, "UNROLL");

  // Copy `bytes` from src to dst (bytes only: every bit pattern is preserved).
  __device__ static __forceinline__ void copy(void* dst, const void* src, size_t bytes) {
    const vec16* s = static_cast<const vec16*>(src);
    vec16* d = static_cast<vec16*>(dst);
    const uint64_t nv = bytes >> 4;
    uint64_t v = threadIdx.x;
    for (; v + (uint64_t)(UNROLL - 1) * THREADS < nv; v += (uint64_t)UNROLL * THREADS) {
      vec16 x[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) x[u] = load16(s + v + (uint64_t)u * THREADS);
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) store16(d + v + (uint64_t)u * THREADS, x[u]);
    }
    for (; v < nv; v += THREADS) store16(d + v, load16(s + v));
  }

  // dst = the ordered reduction of srcs[0..W-1] over `bytes` bytes of element type DT
  // (PLR_BF16, PLR_F16 or PLR_F32), with an optional epilogue. `first_element` is the
  // index of the slice's first element in the caller's numbering (a multiple of the
  // elements per vector); the epilogue sees every vector's own first element and loads
  // by vector index in the same numbering. All W*UNROLL loads of a lane (and the
  // epilogue's) are issued before its first add.
  template <int DT, int W, class Epi = NoEpilogue>
  __device__ static __forceinline__ void reduce(void* dst, const void* const* srcs, size_t bytes,
                                                uint64_t first_element = 0, const Epi& epi = Epi()) {
    static_assert(W >= 1 && W <= PLR_MAX_WORLD, "W");
    constexpr int N = Elems<DT>::N;
    const vec16* s[W];
#pragma unroll
    for (int w = 0; w < W; ++w) s[w] = static_cast<const vec16*>(srcs[w]);
    vec16* d = static_cast<vec16*>(dst);
    const uint64_t nv = bytes >> 4;
    uint64_t v = threadIdx.x;
    const uint64_t first_vec = first_element / N;
    for (; v + (uint64_t)(UNROLL - 1) * THREADS < nv; v += (uint64_t)UNROLL * THREADS) {
      vec16 x[UNROLL][W];
      typename Epi::Pre pre[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
        for (int w = 0; w < W; ++w) x[u][w] = load16(s[w] + v + (uint64_t)u * THREADS);
        pre[u] = epi.load(first_vec + v + (uint64_t)u * THREADS);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const uint64_t vv = v + (uint64_t)u * THREADS;
        store16(d + vv, combine<DT, W, Epi>(x[u], first_element + vv * N, epi, pre[u]));
      }
    }
    for (; v < nv; v += THREADS) {
      vec16 x[W];
#pragma unroll
      for (int w = 0; w < W; ++w) x[w] = load16(s[w] + v);
      const typename Epi::Pre pre = epi.load(first_vec + v);
      store16(d + v, combine<DT, W, Epi>(x, first_element + v * N, epi, pre));
    }
  }
};

// ---- notification (section 3.2) ----
// Publish: every store the calling workgroup made before this call is visible at agent
// scope before `flag` holds `epoch`. Call from all threads of the workgroup.
__device__ __forceinline__ void signal_flag(uint64_t* flag, uint64_t epoch) {
  __syncthreads();  // the workgroup's stores precede the release below
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Consume: lane 0 polls `flag` until it holds at least `epoch` (at most spin_limit
// polls), then acquires; the workgroup barrier hands the acquire to every thread.
// Returns false, on every thread, if the flag did not arrive in time. Call from all
// threads of the workgroup.
__device__ __forceinline__ bool wait_flag(const uint64_t* flag, uint64_t epoch, uint64_t spin_limit) {
  int ok = 1;
  if (threadIdx.x == 0) {
    uint64_t polls = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < epoch) {
      if (++polls >= spin_limit) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  return __syncthreads_and(ok) != 0;
}

// ---- packets (section 3.2 and Figure 7) ----
// The form plr_reduce_packets reads (include/plr.h): a source's packet buffer holds two
// slots of 2 x the share's bytes; the consuming call of epoch e reads slot e & 1, where
// payload word i (4 bytes) of the share is the 8-byte packet at index i, the word in the
// low half and the low 32 bits of e in the high half. e is the layout's epoch plus one
// at the consuming call (plr_layout_epoch(L) + 1).
__host__ __device__ inline uint64_t* packet_slot(void* buffer, uint64_t share_bytes, uint64_t epoch) {
  return reinterpret_cast<uint64_t*>(static_cast<char*>(buffer) + (epoch & 1) * 2 * share_bytes);
}

// Write payload word i of a share into its epoch's slot: one 8-byte atomic store, so the
// consumer never sees the word without its stamp or the stamp without its word. No fence
// is needed: each packet announces only itself.
__device__ __forceinline__ void store_packet(uint64_t* slot, uint64_t i, uint32_t word, uint64_t epoch) {
  __hip_atomic_store(slot + i, ((uint64_t)(uint32_t)epoch << 32) | word, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace atom
}  // namespace plr
