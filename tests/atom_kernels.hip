// User kernels built on the device-callable Atom (include/plr_atom.h), the way the
// project README's "Device-side" samples use it: a kernel of the Atom's THREADS threads
// per workgroup calls copy or reduce on its own slice, fused with its own work. The
// tests load this file's library (tests/libatom_kernels.so) and check every kernel
// against the oracle.
//
//  - atom_block_copy: workgroup b copies bytes [b*per_block, (b+1)*per_block) (the
//    README's copy sample).
//  - atom_block_reduce: workgroup b reduces its slice of W sources; with a residual the
//    epilogue adds it to the binary32 accumulators before the single rounding (an
//    AllReduce fused with a residual add), which is the ordered reduction of the W
//    sources followed by the residual as source W.
//  - atom_pipeline: stage / notify / consume inside one kernel (section 3.2): workgroup
//    b copies chunk b from src to mid and signals its flag, then waits for the flag of
//    chunk b - lag and copies that chunk from mid to dst. Workgroups only wait for
//    lower-numbered ones, which never wait before signalling, and workgroups are
//    dispatched in increasing order, so every wait ends (the tests keep the grid small
//    enough to be resident at once in any case); a bounded wait that gives up records 1
//    in *err and copies nothing.
//  - atom_produce: the producer side of a reduce layout's notified call, written into
//    the producing kernel itself (section 3.2 and Figure 7): workgroup (c, s) produces
//    chunk c of source s's share (here a copy of its input, standing for any producing
//    computation) and either only stores it (mode 0), or stores it and releases the
//    chunk's flag in the layout's workspace (mode 1, signal_flag on flags[s][c]), or
//    writes it as packets of the consuming call's epoch (mode 2, store_packet), which
//    plr_reduce_packets reads with no flag at all.
#include <hip/hip_runtime.h>

#include "plr_atom.h"

using plr::atom::Atom;
using plr::atom::Elems;
using plr::atom::vec16;

namespace {

template <int THREADS>
__global__ void __launch_bounds__(THREADS) k_block_copy(uint8_t* dst, const uint8_t* src, size_t per_block) {
  const size_t off = (size_t)blockIdx.x * per_block;
  Atom<THREADS>::copy(dst + off, src + off, per_block);
}

struct Srcs {
  const uint8_t* p[PLR_MAX_WORLD];
};

// Epilogue: acc += widen(residual vector of the same elements); the residual vector is
// loaded together with the sources' vectors.
template <int DT>
struct AddResidual {
  const vec16* r;
  typedef vec16 Pre;
  __device__ Pre load(uint64_t vec) const { return plr::atom::load16(r + vec); }
  __device__ void operator()(float* acc, int, uint64_t, const Pre& x) const {
    float t[Elems<DT>::N];
    Elems<DT>::widen(x, t);
#pragma unroll
    for (int j = 0; j < Elems<DT>::N; ++j) acc[j] = acc[j] + t[j];
  }
};

template <int DT, int W, int UNROLL>
__global__ void __launch_bounds__(128) k_block_reduce(uint8_t* dst, Srcs s, const uint8_t* residual,
                                                      size_t per_block) {
  constexpr int N = Elems<DT>::N;
  const size_t off = (size_t)blockIdx.x * per_block;
  const void* src[W];
#pragma unroll
  for (int w = 0; w < W; ++w) src[w] = s.p[w] + off;
  const uint64_t first = off / 16 * N;  // element index of the slice's first element
  if (residual)
    Atom<128, UNROLL>::template reduce<DT, W>(dst + off, src, per_block, first,
                                              AddResidual<DT>{reinterpret_cast<const vec16*>(residual)});
  else
    Atom<128, UNROLL>::template reduce<DT, W>(dst + off, src, per_block, first);
}

__global__ void __launch_bounds__(256) k_pipeline(const uint8_t* src, uint8_t* mid, uint8_t* dst, size_t chunk,
                                                  uint32_t nchunks, uint32_t lag, uint64_t* flags,
                                                  uint64_t signal_epoch, uint64_t wait_epoch, uint64_t spin_limit,
                                                  uint32_t* err) {
  const uint32_t b = blockIdx.x;
  if (b < nchunks) {  // stage: produce chunk b, then notify
    Atom<256>::copy(mid + (size_t)b * chunk, src + (size_t)b * chunk, chunk);
    plr::atom::signal_flag(flags + b, signal_epoch);
  }
  if (b >= lag) {  // consume chunk b - lag once its flag has arrived
    const uint32_t c = b - lag;
    if (!plr::atom::wait_flag(flags + c, wait_epoch, spin_limit)) {
      if (threadIdx.x == 0) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    Atom<256>::copy(dst + (size_t)c * chunk, mid + (size_t)c * chunk, chunk);
  }
}

struct ProduceArgs {
  const uint8_t* in[PLR_MAX_WORLD];
  void* out[PLR_MAX_WORLD];  // mode 0 / 1: the share; mode 2: the packet buffer
  uint64_t share, chunk;     // bytes of a share, bytes per chunk (one workgroup each)
  uint64_t* flags;           // mode 1: flags[s][c], nchunks per source
  uint32_t nchunks;
  uint64_t epoch;            // the consuming call's epoch
};

template <int MODE>
__global__ void __launch_bounds__(256) k_produce(const ProduceArgs a) {
  constexpr int T = 256;
  const uint32_t c = blockIdx.x, s = blockIdx.y;
  const uint64_t off = (uint64_t)c * a.chunk;
  const uint64_t len = min(a.chunk, a.share - off);
  if (MODE < 2) {
    Atom<T>::copy(static_cast<uint8_t*>(a.out[s]) + off, a.in[s] + off, len);
    if (MODE == 1) plr::atom::signal_flag(a.flags + (uint64_t)s * a.nchunks + c, a.epoch);
  } else {
    uint64_t* slot = plr::atom::packet_slot(a.out[s], a.share, a.epoch);
    const uint32_t* in = reinterpret_cast<const uint32_t*>(a.in[s] + off);
    const uint64_t w0 = off / 4, nw = len / 4;
    uint64_t i = threadIdx.x;
    for (; i + 3 * T < nw; i += 4 * T) {  // four words per lane in flight
      uint32_t x[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = __builtin_nontemporal_load(in + i + k * T);
#pragma unroll
      for (int k = 0; k < 4; ++k) plr::atom::store_packet(slot, w0 + i + k * T, x[k], a.epoch);
    }
    for (; i < nw; i += T) plr::atom::store_packet(slot, w0 + i, __builtin_nontemporal_load(in + i), a.epoch);
  }
}

template <int DT, int W>
hipError_t launch_reduce_u(int unroll, uint8_t* dst, const Srcs& s, const uint8_t* residual, size_t per_block,
                           uint32_t nblocks, hipStream_t st) {
  if (unroll == 2)
    hipLaunchKernelGGL((k_block_reduce<DT, W, 2>), dim3(nblocks), dim3(128), 0, st, dst, s, residual, per_block);
  else
    hipLaunchKernelGGL((k_block_reduce<DT, W, 1>), dim3(nblocks), dim3(128), 0, st, dst, s, residual, per_block);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_reduce_w(int world, int unroll, uint8_t* dst, const Srcs& s, const uint8_t* residual,
                           size_t per_block, uint32_t nblocks, hipStream_t st) {
  switch (world) {
    case 1: return launch_reduce_u<DT, 1>(unroll, dst, s, residual, per_block, nblocks, st);
    case 2: return launch_reduce_u<DT, 2>(unroll, dst, s, residual, per_block, nblocks, st);
    case 3: return launch_reduce_u<DT, 3>(unroll, dst, s, residual, per_block, nblocks, st);
    case 8: return launch_reduce_u<DT, 8>(unroll, dst, s, residual, per_block, nblocks, st);
    default: return hipErrorInvalidValue;
  }
}

bool a16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

// Host launchers: argument checks on the host, then one launch. Return a hipError_t.
extern "C" int atom_block_copy(void* dst, const void* src, size_t per_block, unsigned nblocks, int threads,
                               void* stream) {
  if (!dst || !src || !nblocks || (per_block & 15) || !a16(dst) || !a16(src)) return (int)hipErrorInvalidValue;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* d = static_cast<uint8_t*>(dst);
  const uint8_t* s = static_cast<const uint8_t*>(src);
  switch (threads) {
    case 64: hipLaunchKernelGGL(k_block_copy<64>, dim3(nblocks), dim3(64), 0, st, d, s, per_block); break;
    case 128: hipLaunchKernelGGL(k_block_copy<128>, dim3(nblocks), dim3(128), 0, st, d, s, per_block); break;
    case 256: hipLaunchKernelGGL(k_block_copy<256>, dim3(nblocks), dim3(256), 0, st, d, s, per_block); break;
    case 512: hipLaunchKernelGGL(k_block_copy<512>, dim3(nblocks), dim3(512), 0, st, d, s, per_block); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

extern "C" int atom_block_reduce(int dtype, int world, const void* const* srcs, const void* residual, void* dst,
                                 size_t per_block, unsigned nblocks, int unroll, void* stream) {
  if (!srcs || !dst || !nblocks || (per_block & 15) || !a16(dst) || world < 1 || world > PLR_MAX_WORLD)
    return (int)hipErrorInvalidValue;
  if (residual && !a16(residual)) return (int)hipErrorInvalidValue;
  Srcs s{};
  for (int w = 0; w < world; ++w) {
    if (!srcs[w] || !a16(srcs[w])) return (int)hipErrorInvalidValue;
    s.p[w] = static_cast<const uint8_t*>(srcs[w]);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* d = static_cast<uint8_t*>(dst);
  const uint8_t* r = static_cast<const uint8_t*>(residual);
  switch (dtype) {
    case PLR_BF16: return (int)launch_reduce_w<PLR_BF16>(world, unroll, d, s, r, per_block, nblocks, st);
    case PLR_F16: return (int)launch_reduce_w<PLR_F16>(world, unroll, d, s, r, per_block, nblocks, st);
    case PLR_F32: return (int)launch_reduce_w<PLR_F32>(world, unroll, d, s, r, per_block, nblocks, st);
    default: return (int)hipErrorInvalidValue;
  }
}

// signal_epoch is what producers store, wait_epoch what consumers wait for (equal in
// normal use; a smaller signal_epoch makes every bounded wait give up).
extern "C" int atom_pipeline(const void* src, void* mid, void* dst, size_t chunk, unsigned nchunks, unsigned lag,
                             void* flags, unsigned long long signal_epoch, unsigned long long wait_epoch,
                             unsigned long long spin_limit, void* err, void* stream) {
  if (!src || !mid || !dst || !flags || !err || !nchunks || !lag || (chunk & 15) || !a16(src) || !a16(mid) ||
      !a16(dst) || ((uintptr_t)flags & 7) || ((uintptr_t)err & 3))
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_pipeline, dim3(nchunks + lag), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(src), static_cast<uint8_t*>(mid), static_cast<uint8_t*>(dst), chunk,
                     (uint32_t)nchunks, (uint32_t)lag, static_cast<uint64_t*>(flags), (uint64_t)signal_epoch,
                     (uint64_t)wait_epoch, (uint64_t)spin_limit, static_cast<uint32_t*>(err));
  return (int)hipGetLastError();
}

// mode 0: store only; 1: store, then release flags[s][c] (flags = the workspace's flag
// array, nchunks = ceil(share / chunk)); 2: packets into out[s] (packet buffers).
extern "C" int atom_produce(int mode, int world, const void* const* in, void* const* out, size_t share, size_t chunk,
                            void* flags, unsigned long long epoch, void* stream) {
  if (mode < 0 || mode > 2 || !in || !out || world < 1 || world > PLR_MAX_WORLD || !share || !chunk ||
      (share & 15) || (chunk & 15) || (mode == 1 && (!flags || ((uintptr_t)flags & 7))))
    return (int)hipErrorInvalidValue;
  const uint64_t nchunks = (share + chunk - 1) / chunk;
  if (nchunks > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
  ProduceArgs a{};
  for (int w = 0; w < world; ++w) {
    if (!in[w] || !out[w] || !a16(in[w]) || !a16(out[w])) return (int)hipErrorInvalidValue;
    a.in[w] = static_cast<const uint8_t*>(in[w]);
    a.out[w] = out[w];
  }
  a.share = share;
  a.chunk = chunk;
  a.flags = static_cast<uint64_t*>(flags);
  a.nchunks = (uint32_t)nchunks;
  a.epoch = epoch;
  const dim3 g((uint32_t)nchunks, (uint32_t)world), b(256);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: hipLaunchKernelGGL(k_produce<0>, g, b, 0, st, a); break;
    case 1: hipLaunchKernelGGL(k_produce<1>, g, b, 0, st, a); break;
    default: hipLaunchKernelGGL(k_produce<2>, g, b, 0, st, a); break;
  }
  return (int)hipGetLastError();
}
