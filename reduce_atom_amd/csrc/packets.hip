// Latency path: payload and notification in one atomic packet.
//
// Purlin paper, section 3.2 (and Figure 7): for latency-bound transfers the producer
// pushes packets that carry the payload together with the notification, so the
// consumer needs no separate flag round trip, at the price of doubling the data
// volume; section 3.3: the packets are still reduced element by element, in source
// order. On gfx950 the single-copy-atomic unit is 8 bytes, so a packet is a 4-byte
// payload word in the low half and the low 32 bits of the epoch in the high half,
// written with one 8-byte atomic store and read with one 8-byte atomic load. A packet
// carries its own data, so the consumer needs no acquire fence.
//
// Access pattern: a wave owns a group of 4 x 64 consecutive payload words and lane l
// handles words l, l+64, l+128 and l+192 of it, so every 8-byte packet access and
// every 4-byte payload access of a wave is one contiguous run (512 or 256 bytes). The
// reduction is elementwise, so which words share a lane does not matter.
#include "device_common.h"

namespace plr {

constexpr int kPacketBlock = 128;
constexpr uint64_t kWaveWords = 256;

__device__ __forceinline__ uint64_t wave_base() {
  return ((uint64_t)blockIdx.x * kPacketBlock + threadIdx.x) / 64 * kWaveWords + (threadIdx.x & 63);
}

// Producer: source blockIdx.y of the launch stamps its share into its packets.
__global__ void __launch_bounds__(kPacketBlock) k_pack(const PackArgs a) {
  const uint32_t s = a.first + blockIdx.y;
  const uint32_t* data = a.data[s];
  uint64_t* pk = a.packets[s];
  const uint64_t base = wave_base();
  uint32_t x[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t i = base + 64 * k;
    if (i < a.nwords) x[k] = __builtin_nontemporal_load(data + i);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t i = base + 64 * k;
    if (i < a.nwords) atom::store_packet(pk, i, x[k], a.stamp);
  }
}

// Consumer: load the W x 4 packets of the lane, re-poll only those whose stamp is not
// yet the epoch's (bounded), then reduce the payloads in source order.
template <int DT, int W>
__global__ void __launch_bounds__(kPacketBlock) k_reduce_packets(const PacketReduceArgs a) {
  const uint64_t base = wave_base();
  if (base >= a.nwords) return;
  bool live[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) live[k] = base + 64 * k < a.nwords;
  uint64_t p[W][4];
#pragma unroll
  for (int w = 0; w < W; ++w)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      p[w][k] = live[k] ? __hip_atomic_load(a.pk[w] + base + 64 * k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        : (uint64_t)a.stamp << 32;
  uint64_t polls = 0;
  while (true) {
    bool all = true;
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if ((uint32_t)(p[w][k] >> 32) != a.stamp) {
          all = false;
          p[w][k] = __hip_atomic_load(a.pk[w] + base + 64 * k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    if (all) break;
    if (++polls >= a.spin_limit) {
      uint64_t expect = 0;
      __hip_atomic_compare_exchange_strong(a.err, &expect, (uint64_t)PLR_ETIMEOUT, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  u32x4 x[W];
#pragma unroll
  for (int w = 0; w < W; ++w)
    x[w] = (u32x4){(uint32_t)p[w][0], (uint32_t)p[w][1], (uint32_t)p[w][2], (uint32_t)p[w][3]};
  const u32x4 y = combine<DT, W>(x);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (live[k]) __builtin_nontemporal_store(y[k], a.dst + base + 64 * k);
}

static dim3 packet_grid(uint64_t nwords, uint32_t y) {
  const uint64_t waves = (nwords + kWaveWords - 1) / kWaveWords;
  const uint64_t blocks = (waves + kPacketBlock / 64 - 1) / (kPacketBlock / 64);
  return dim3((uint32_t)(blocks ? blocks : 1), y);
}

hipError_t launch_pack(const PackArgs& a, uint32_t nsrc, hipStream_t s) {
  hipLaunchKernelGGL(k_pack, packet_grid(a.nwords, nsrc), dim3(kPacketBlock), 0, s, a);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_rp_dt(const PacketReduceArgs& a, hipStream_t s) {
  const dim3 g = packet_grid(a.nwords, 1), b(kPacketBlock);
  switch (a.world) {
#define PLR_W(w)                                                         \
  case w:                                                                \
    launch_dp(k_reduce_packets<DT, w>, g, b, 0, s, true, true, a);        \
    return hipGetLastError();
    PLR_W(1) PLR_W(2) PLR_W(3) PLR_W(4) PLR_W(5) PLR_W(6) PLR_W(7) PLR_W(8)
    PLR_W(9) PLR_W(10) PLR_W(11) PLR_W(12) PLR_W(13) PLR_W(14) PLR_W(15) PLR_W(16)
#undef PLR_W
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_reduce_packets(const PacketReduceArgs& a, int dtype, hipStream_t s) {
  switch (dtype) {
    case PLR_BF16: return launch_rp_dt<PLR_BF16>(a, s);
    case PLR_F16: return launch_rp_dt<PLR_F16>(a, s);
    case PLR_F32: return launch_rp_dt<PLR_F32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace plr
