// Device helpers shared by the kernels: 16-byte vector access, element conversions,
// and the consumer side of chunk notification.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "plr_atom.h"

namespace plr {

// Streaming 16-byte access, element conversions and the ordered combine come from the
// device-callable Atom (include/plr_atom.h), so the library's kernels and user kernels
// that call the Atom run the same code.
__device__ __forceinline__ u32x4 ld16(const u32x4* p) { return atom::load16(p); }
__device__ __forceinline__ void st16(u32x4* p, u32x4 v) { atom::store16(p, v); }
using atom::combine;
using atom::Elems;

// Launch of a datapath kernel: `first` / `last` say whether it opens / closes the
// call's datapath, which decides which of the thread's timing events it carries. `lds`
// bytes of workgroup memory are reserved per workgroup beyond the kernel's own; no kernel
// touches them: they only bound how many workgroups a compute unit holds at once.
template <typename K, typename... A>
inline void launch_dp(K kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, bool first, bool last,
                      A... args) {
  const Timing& t = timing();
  hipEvent_t a = first ? t.start : (last ? t.last_start : nullptr);
  hipEvent_t b = last ? t.stop : (first ? t.first_stop : nullptr);
  hipExtLaunchKernelGGL(kernel, grid, block, lds, s, a, b, 0, args...);
}

// Constant address space: loads through such a pointer that are the same for every
// lane become scalar loads. Only for data that no kernel writes while the reading
// kernel runs (the scalar cache is refilled at every kernel start).
#define PLR_CONST __attribute__((address_space(4)))

// ---- XCD-aware workgroup order ----
// The dispatcher hands workgroup b to XCD b % 8 (MI355X has 8 XCDs, each with its
// own L2). When `xcd` is set, logical workgroup ids are renumbered so that each XCD
// runs one contiguous range of them: XCD x gets ids [x*q + min(x, r), ...) where
// q, r = grid / 8, grid % 8. This is a bijection on [0, grid). Measured on MI355X: a
// kernel that only reads 8 streams ran 10% faster this way, but the reduce and the
// copies, which also write, ran 1-8% slower, so the layouts' policy leaves it off and
// it stays an option (xcd_order).
constexpr uint32_t kXcds = 8;

__device__ __forceinline__ uint32_t logical_block(int xcd) {
  const uint32_t b = blockIdx.x;
  if (!xcd) return b;
  const uint32_t G = gridDim.x, q = G / kXcds, r = G % kXcds;
  const uint32_t x = b % kXcds, k = b / kXcds;
  return x * q + min(x, r) + k;
}

// ---- consumer side of notify (section 3.2) ----
// Lanes 0..n-1 of the calling wave each own one flag, index first + lane*stride in the
// layout's flag array. A lane whose flag the check kernel already saw arrive (mirror,
// check mode) needs nothing more: that kernel's acquire and the kernel boundary order
// this kernel after the producer. Otherwise the lane polls the flag until it reaches
// nt.epoch, within a bounded number of polls, and the wave then executes one
// agent-scope acquire fence. On a timeout one lane records PLR_ETIMEOUT in the sticky
// error word; if another wave already recorded an error the wave gives up too. A wait
// that found some flag below the epoch at its first poll adds one to the workspace's
// late counter (header word 2), so that a caller can tell consumers that waited from
// those that found their data announced. Returns true when every flag has arrived. All
// lanes of the wave call this together.
__device__ __forceinline__ bool wait_flags(const Notify& nt, uint64_t first, uint64_t stride, int n) {
  const int lane = __lane_id();
  int bad = 0, polled = 0, late = 0;
  if (lane < n) {
    const uint64_t i = first + (uint64_t)lane * stride;
    if (!(nt.mirror && nt.mirror[i] == nt.epoch)) {
      polled = 1;
      const uint64_t* f = nt.flags + i;
      uint64_t polls = 0;
      while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nt.epoch) {
        late = 1;
        if (++polls >= nt.spin_limit) {
          bad = 1;
          break;
        }
        if ((polls & 63) == 0 &&
            __hip_atomic_load(nt.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
          bad = 2;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
  }
  const uint64_t timed_out = __ballot(bad == 1);
  const uint64_t failed = __ballot(bad != 0);
  const uint64_t waited = __ballot(late);
  if (waited && lane == __builtin_ctzll(waited))
    __hip_atomic_fetch_add(nt.err + kLateWord, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (failed) {
    if (timed_out && lane == __builtin_ctzll(timed_out)) {
      uint64_t expect = 0;
      __hip_atomic_compare_exchange_strong(nt.err, &expect, (uint64_t)PLR_ETIMEOUT, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return false;
  }
  if (__ballot(polled)) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

// True when the call must look at chunk flags itself: it is notified and the check
// kernel that ran before it (stream order) did not find every flag already arrived.
__device__ __forceinline__ bool must_wait(const Notify& nt) {
  return nt.flags && !(nt.ready && *nt.ready == nt.epoch);
}

// Workgroup form: only wave 0 polls and executes the agent-scope acquire (on a chip
// with one L2 per XCD that acquire invalidates cached lines, so it is paid once per
// workgroup and chunk, not once per wave); the workgroup barrier then orders the
// other waves' loads after it. Returns false on a timeout or an earlier error. Every
// thread of the workgroup must call this together.
__device__ __forceinline__ bool wg_wait_flags(const Notify& nt, uint64_t first, uint64_t stride, int n) {
  const bool ok = (threadIdx.x >> 6) ? true : wait_flags(nt, first, stride, n);
  return !__syncthreads_or(!ok);
}

}  // namespace plr

namespace plr {

// ---- LDS staging (the Atom pipeline through workgroup-local memory) ----
// gfx950 global->LDS DMA: each lane's 16 bytes land at lds_base + 16*lane, where
// lds_base is wave-uniform. The LDS reads that consume a stage are inline ds_read_b128
// with their own wait (lds_read_wait), so that the compiler does not wait for every
// DMA in flight (it cannot tell the stages of the ring apart) and the pipeline keeps
// S-1 stages loading while one is consumed.
#define PLR_LDS __attribute__((address_space(3)))

__device__ __forceinline__ void lds_dma16(const void* gsrc, PLR_LDS void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_base, 16, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding. Loads
// complete in issue order, so once at most N operations are outstanding every load
// issued before the last N memory operations has landed (stores issued in between
// only make the wait stricter).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS reads of a ring slab and their wait in one assembly statement: out[k] = the 16-byte
// vector at `base` + k KiB, k < N, all N reads in flight together, then a wait for them.
// The compiler takes an assembly statement's outputs as written when the statement
// ends, so with the reads and the wait in separate statements it may schedule uses of
// the outputs between them (a reduce's widening was placed right after the read, before
// the data had arrived). The outputs are early-clobber: none may share a register with
// the address, which the later reads of the statement still use. Groups of at most 8
// (the immediate offsets stay under 8 KiB); more than 8 take one statement per group.
template <int N>
struct LdsReadWait;
template <>
struct LdsReadWait<1> {
  static __device__ __forceinline__ void run(uint32_t a, u32x4* o) {
    asm volatile(
        "ds_read_b128 %0, %1\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0])
        : "v"(a)
        : "memory");
  }
};
template <>
struct LdsReadWait<2> {
  static __device__ __forceinline__ void run(uint32_t a, u32x4* o) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %2 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1])
        : "v"(a)
        : "memory");
  }
};
template <>
struct LdsReadWait<3> {
  static __device__ __forceinline__ void run(uint32_t a, u32x4* o) {
    asm volatile(
        "ds_read_b128 %0, %3\n\t"
        "ds_read_b128 %1, %3 offset:1024\n\t"
        "ds_read_b128 %2, %3 offset:2048\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2])
        : "v"(a)
        : "memory");
  }
};
template <>
struct LdsReadWait<4> {
  static __device__ __forceinline__ void run(uint32_t a, u32x4* o) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\t"
        "ds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
        : "v"(a)
        : "memory");
  }
};
template <>
struct LdsReadWait<5> {
  static __device__ __forceinline__ void run(uint32_t a, u32x4* o) {
    asm volatile(
        "ds_read_b128 %0, %5\n\t"
        "ds_read_b128 %1, %5 offset:1024\n\t"
        "ds_read_b128 %2, %5 offset:2048\n\t"
        "ds_read_b128 %3, %5 offset:3072\n\t"
        "ds_read_b128 %4, %5 offset:4096\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4])
        : "v"(a)
        : "memory");
  }
};
template <>
struct LdsReadWait<6> {
  static __device__ __forceinline__ void run(uint32_t a, u32x4* o) {
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %6 offset:1024\n\t"
        "ds_read_b128 %2, %6 offset:2048\n\t"
        "ds_read_b128 %3, %6 offset:3072\n\t"
        "ds_read_b128 %4, %6 offset:4096\n\t"
        "ds_read_b128 %5, %6 offset:5120\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5])
        : "v"(a)
        : "memory");
  }
};
template <>
struct LdsReadWait<7> {
  static __device__ __forceinline__ void run(uint32_t a, u32x4* o) {
    asm volatile(
        "ds_read_b128 %0, %7\n\t"
        "ds_read_b128 %1, %7 offset:1024\n\t"
        "ds_read_b128 %2, %7 offset:2048\n\t"
        "ds_read_b128 %3, %7 offset:3072\n\t"
        "ds_read_b128 %4, %7 offset:4096\n\t"
        "ds_read_b128 %5, %7 offset:5120\n\t"
        "ds_read_b128 %6, %7 offset:6144\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6])
        : "v"(a)
        : "memory");
  }
};
template <>
struct LdsReadWait<8> {
  static __device__ __forceinline__ void run(uint32_t a, u32x4* o) {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\t"
        "ds_read_b128 %3, %8 offset:3072\n\t"
        "ds_read_b128 %4, %8 offset:4096\n\t"
        "ds_read_b128 %5, %8 offset:5120\n\t"
        "ds_read_b128 %6, %8 offset:6144\n\t"
        "ds_read_b128 %7, %8 offset:7168\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
        : "v"(a)
        : "memory");
  }
};

template <int N>
__device__ __forceinline__ void lds_read_wait(const PLR_LDS u32x4* base, u32x4* out) {
  static_assert(N >= 1, "at least one vector");
  if constexpr (N > 8) {
    LdsReadWait<8>::run((uint32_t)(uintptr_t)base, out);
    lds_read_wait<N - 8>(base + 8 * 64, out + 8);
  } else {
    LdsReadWait<N>::run((uint32_t)(uintptr_t)base, out);
  }
}

}  // namespace plr
