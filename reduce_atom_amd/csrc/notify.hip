// Producer side of notify (Purlin paper, section 3.2 "SNAC": a stage is announced by
// a flag; section 4.3 "Epoch Bookkeeping": a monotonic 64-bit epoch supplies the
// value). One release fence per wave orders everything this stream already did
// before the flag stores, which are agent-scope atomics so that consumers on any
// XCD observe them.
#include "device_common.h"

namespace plr {

__global__ void __launch_bounds__(256) k_notify(const NotifyArgs a) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.nflags; i += stride)
    __hip_atomic_store(a.flags + i, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Check ahead of a notified consumer: it reads every chunk flag once (agent-scope
// atomic loads), mirrors which ones have reached the epoch, and if all have it records
// the epoch in the workspace's ready word. The acquire fence makes the producers'
// releases happen before this kernel's end, so the consuming kernel that follows in
// stream order may read every chunk whose flag was mirrored without waiting or
// fencing; only the chunks still missing are waited for one by one (section 3.2: a
// consumer never reads a chunk before its flag). One workgroup does it all, with
// kCheckUnroll flag loads per lane in flight, so that the outcome needs one round of
// loads and a workgroup barrier, not a second kernel-wide combining step.
constexpr int kCheckUnroll = 8;

__global__ void __launch_bounds__(kCheckThreads) k_check(const CheckArgs a) {
  int ok = 1;
  for (uint64_t base = 0; base < a.nflags; base += (uint64_t)kCheckThreads * kCheckUnroll) {
    uint64_t f[kCheckUnroll];
#pragma unroll
    for (int u = 0; u < kCheckUnroll; ++u) {
      const uint64_t i = base + (uint64_t)u * kCheckThreads + threadIdx.x;
      f[u] = i < a.nflags ? __hip_atomic_load(a.flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : a.epoch;
    }
#pragma unroll
    for (int u = 0; u < kCheckUnroll; ++u) {
      const uint64_t i = base + (uint64_t)u * kCheckThreads + threadIdx.x;
      const bool arrived = f[u] >= a.epoch;
      if (i < a.nflags) a.mirror[i] = arrived ? a.epoch : 0;
      ok &= arrived;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int all = __syncthreads_and(ok);
  if (threadIdx.x == 0) *a.ready = all ? a.epoch : 0;
}

hipError_t launch_check(const CheckArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_check, dim3(1), dim3(kCheckThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_notify(const NotifyArgs& a, hipStream_t s) {
  uint64_t blocks = (a.nflags + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 256) blocks = 256;
  hipLaunchKernelGGL(k_notify, dim3((uint32_t)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace plr
