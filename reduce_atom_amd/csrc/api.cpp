// C ABI entry points: validation, kernel argument marshalling, launch, epoch advance.
// Every step of the datapath runs in the HIP kernels; this file only checks
// arguments on the host and fills the kernel argument blocks.
#include <hip/hip_runtime_api.h>

#include <algorithm>

#include "kernels.h"
#include "layout.h"

using namespace plr;

namespace {

thread_local int g_last_hip = 0;

thread_local Timing g_timing = {nullptr, nullptr, nullptr, nullptr};

int hip_fail(hipError_t e) { return plr::record_hip_error(e); }

bool a16(const void* p) { return ((uintptr_t)p & 15) == 0; }

bool overlaps(uintptr_t a0, uint64_t alen, uintptr_t b0, uint64_t blen) {
  return alen && blen && a0 < b0 + blen && b0 < a0 + alen;
}

// Tiles of a call: notified calls use the chunk-aligned shape, un-notified ones the
// layout's plain shape (the same except for latency-regime reduces).
uint64_t tiles_of(const plr_layout* L, bool notified) {
  return notified ? L->ntiles : L->plain_ntiles;
}

// Tiles per workgroup: the policy's run, or what an explicit workgroup count implies;
// the grid then covers every tile once.
uint32_t run_for(const plr_layout* L, bool notified) {
  uint64_t g = 0;
  if (L->workgroups > 0) g = (uint64_t)L->workgroups;
  if (g == 0) return (uint32_t)std::max(1, notified ? L->run_notified : L->run);
  return (uint32_t)std::max<uint64_t>(1, (tiles_of(L, notified) + g - 1) / g);
}

Launch launch_of(const plr_layout* L, bool notified) {
  const uint32_t run = run_for(L, notified);
  const uint32_t grid = (uint32_t)std::max<uint64_t>(1, (tiles_of(L, notified) + run - 1) / run);
  const int xcd = L->xcd_order == kXcdOn;
  const uint32_t block = (uint32_t)(notified ? L->block : L->plain_block);
  return Launch{grid, block, L->unroll, L->stages, L->datapath, run, xcd, L->lds_reserve};
}

// Common checks of plr_reduce / plr_copy. Fills the notification block.
int check_call(const plr_layout* L, plr_op op, const void* const* srcs, const void* dst,
               void* workspace, Notify* nt) {
  if (!L || L->op != op || !srcs || !dst) return PLR_EINVAL;
  if (L->datapath == PLR_PATH_COMPOSED) return PLR_EINVAL;
  if (!a16(dst)) return PLR_EALIGN;
  for (int w = 0; w < L->world; ++w) {
    if (!srcs[w]) return PLR_EINVAL;
    if (!a16(srcs[w])) return PLR_EALIGN;
  }
  // the output must not overlap anything the call reads
  for (const auto& s : L->segs)
    if (overlaps((uintptr_t)dst, L->dst_bytes, (uintptr_t)srcs[s.src] + s.src_off, s.len))
      return PLR_EINVAL;
  nt->flags = nullptr;
  nt->err = nullptr;
  nt->epoch = L->epoch + 1;
  nt->spin_limit = L->spin_limit;
  nt->ready = nullptr;
  nt->mirror = nullptr;
  if (workspace) {
    if (!a16(workspace)) return PLR_EALIGN;
    nt->err = static_cast<uint64_t*>(workspace);
    nt->flags = reinterpret_cast<const uint64_t*>(static_cast<char*>(workspace) + kWorkspaceHeader);
    if (L->notify_mode == PLR_NOTIFY_CHECK) {
      nt->ready = static_cast<uint64_t*>(workspace) + 1;
      nt->mirror = nt->flags + nflags(L);
    }
  }
  return PLR_OK;
}

// The check kernel of a notified call in PLR_NOTIFY_CHECK mode.
hipError_t launch_check_for(const plr_layout* L, const Notify& nt, hipStream_t s) {
  if (!nt.ready || !L->ntiles) return hipSuccess;
  CheckArgs c{};
  c.flags = nt.flags;
  c.nflags = nflags(L);
  c.epoch = nt.epoch;
  c.ready = const_cast<uint64_t*>(nt.ready);
  c.mirror = const_cast<uint64_t*>(nt.mirror);
  return launch_check(c, s);
}

}  // namespace

const Timing& plr::timing() { return g_timing; }

int plr::record_hip_error(hipError_t e) {
  g_last_hip = (int)e;
  return PLR_EHIP;
}

extern "C" int plr_reduce(plr_layout* L, const void* const* srcs, void* dst, void* workspace,
                          void* stream) {
  Notify nt;
  int rc = check_call(L, PLR_OP_REDUCE, srcs, dst, workspace, &nt);
  if (rc) return rc;
  if (L->ntiles) {
    ReduceArgs a{};
    for (int w = 0; w < L->world; ++w)
      a.src[w] = reinterpret_cast<const u32x4*>(static_cast<const char*>(srcs[w]) + L->segs[w].src_off);
    const bool notified = nt.flags != nullptr;
    a.dst = static_cast<u32x4*>(dst);
    a.nvec = L->seg_len / 16;
    a.tile_vecs = (notified ? L->tile_bytes : L->plain_tile_bytes) / 16;
    a.ntiles = (uint32_t)tiles_of(L, notified);
    a.tiles_per_chunk = L->tiles_per_chunk;
    a.nchunks = L->nchunks;
    a.world = (uint32_t)L->world;
    a.nt = nt;
    const Launch l = launch_of(L, notified);
    a.run = l.run;
    a.xcd = (uint32_t)l.xcd;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_check_for(L, nt, s);
    if (e == hipSuccess) e = launch_reduce(a, L->dtype, l, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (workspace) L->epoch = nt.epoch;
  return PLR_OK;
}

extern "C" int plr_copy(plr_layout* L, const void* const* srcs, void* dst, void* workspace,
                        void* stream) {
  Notify nt;
  int rc = check_call(L, PLR_OP_COPY, srcs, dst, workspace, &nt);
  if (rc) return rc;
  if (L->ntiles) {
    CopyArgs a{};
    for (int w = 0; w < L->world; ++w) a.src[w] = static_cast<const uint8_t*>(srcs[w]);
    a.dst = static_cast<uint8_t*>(dst);
    a.seg_len = L->seg_len;
    a.tile_bytes = L->tile_bytes;
    a.tiles_per_seg = L->tiles_per_seg;
    a.ntiles = L->ntiles;
    a.tiles_per_chunk = L->tiles_per_chunk;
    a.chunks_per_seg = L->chunks_per_seg;
    a.nchunks = L->nchunks;
    a.nseg = (uint32_t)L->segs.size();
    a.world = (uint32_t)L->world;
    a.nt = nt;
    if (L->table_fits) {
      a.mode = kCopyTable;
      for (size_t k = 0; k < L->segs.size(); ++k) {
        a.seg_src[k] = (uint32_t)L->segs[k].src;
        a.seg_src_off[k] = L->segs[k].src_off;
        a.seg_dst_off[k] = L->segs[k].dst_off;
      }
    } else {  // only derived AllToAll tables exceed the kernarg table
      a.mode = kCopyTransposed;
      a.slice = L->seg_len;
    }
    if (L->var_segs) {  // AllGatherV: segments of their own lengths (at most W of them)
      a.mode = kCopyVar;
      for (int k = 0; k <= PLR_MAX_WORLD; ++k) a.var_tile0[k] = ~0u;
      for (size_t k = 0; k < L->segs.size(); ++k) {
        a.var_tile0[k] = L->seg_tile0[k];
        a.var_chunk0[k] = L->seg_chunk0[k];
        a.var_len[k] = L->segs[k].len;
        a.var_shift[k] = L->seg_shift[k];
      }
      a.var_tile0[L->segs.size()] = L->seg_tile0[L->segs.size()];
      a.var_chunk0[L->segs.size()] = L->seg_chunk0[L->segs.size()];
    }
    const Launch l = launch_of(L, nt.flags != nullptr);
    a.run = l.run;
    a.xcd = (uint32_t)l.xcd;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_check_for(L, nt, s);
    if (e == hipSuccess) e = launch_copy(a, l, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (workspace) L->epoch = nt.epoch;
  return PLR_OK;
}

// Scratch of plr_copy_v: a 256-byte header (u32 ticket at byte 0), uint32 key[rows],
// then int32 seg_count[segments][W] and int32 seg_out[segments][PLR_MAX_WORLD], each
// region rounded up to 256 bytes; a segment is kRankSeg rows of one source.
constexpr uint64_t kCopyVScratchHeader = 256;

static uint64_t up256(uint64_t x) { return (x + 255) & ~255ull; }

int plr::copy_v_check_rows(int world, const int64_t* rows_per_src) {
  if (!rows_per_src) return PLR_EINVAL;
  int64_t total = 0;
  for (int s = 0; s < world; ++s) {
    if (rows_per_src[s] < 0) return PLR_EINVAL;
    if (rows_per_src[s] > 0x7FFFFFFF) return PLR_EUNSUPPORTED;
    total += rows_per_src[s];  // at most 16 x (2^31 - 1): no overflow
  }
  return total > 0x7FFFFFFF ? PLR_EUNSUPPORTED : PLR_OK;
}

struct CopyVScratch {
  uint64_t key_off, count_off, out_off, bytes;
};

static CopyVScratch copy_v_scratch(int world, const int64_t* rows_per_src) {
  uint64_t total = 0, segs = 0;
  for (int s = 0; s < world; ++s) {
    const uint64_t r = rows_per_src[s] > 0 ? (uint64_t)rows_per_src[s] : 0;
    total += r;
    segs += (r + kRankSeg - 1) / kRankSeg;
  }
  CopyVScratch c;
  c.key_off = kCopyVScratchHeader;
  c.count_off = c.key_off + up256(total * sizeof(uint32_t));
  c.out_off = c.count_off + up256(segs * world * sizeof(int32_t));
  c.bytes = c.out_off + up256(segs * PLR_MAX_WORLD * sizeof(int32_t));
  return c;
}

extern "C" size_t plr_copy_v_scratch_bytes(int world, const int64_t* rows_per_src) {
  if (world < 1 || world > PLR_MAX_WORLD) return 0;
  if (copy_v_check_rows(world, rows_per_src) != PLR_OK) return 0;
  return (size_t)copy_v_scratch(world, rows_per_src).bytes;
}

extern "C" int plr_copy_v(int world, const void* const* srcs, const int64_t* rows_per_src,
                          const int32_t* const* dest_of_row, size_t row_bytes, void* dst,
                          int64_t* counts, int64_t* offsets, void* scratch, void* stream) {
  if (world < 1) return PLR_EINVAL;
  if (world > PLR_MAX_WORLD) return PLR_EUNSUPPORTED;
  if (!srcs || !rows_per_src || !dest_of_row || !counts || !offsets || !scratch) return PLR_EINVAL;
  if (row_bytes == 0) return PLR_EINVAL;
  if (row_bytes % 16) return PLR_EALIGN;
  if (((uintptr_t)counts & 7) || ((uintptr_t)offsets & 7) || !a16(scratch)) return PLR_EALIGN;
  const int rows_rc = copy_v_check_rows(world, rows_per_src);
  if (rows_rc != PLR_OK) return rows_rc;
  CopyVArgs a{};
  a.row_start[0] = 0;
  for (int s = 0; s < world; ++s) {
    if (rows_per_src[s] > 0) {
      if (!srcs[s] || !dest_of_row[s] || !dst) return PLR_EINVAL;
      if (!a16(srcs[s])) return PLR_EALIGN;
      if ((uintptr_t)dest_of_row[s] & 3) return PLR_EALIGN;
    }
    a.src[s] = static_cast<const uint8_t*>(srcs[s]);
    a.dest[s] = dest_of_row[s];
    a.row_start[s + 1] = a.row_start[s] + rows_per_src[s];
  }
  const int64_t total = a.row_start[world];
  for (int s = world + 1; s <= PLR_MAX_WORLD; ++s) a.row_start[s] = total;
  if (total > 0) {
    // an output past 2^64 bytes cannot exist (and would wrap the overlap check)
    if (row_bytes > UINT64_MAX / (uint64_t)total) return PLR_EINVAL;
    if (!a16(dst)) return PLR_EALIGN;
    const uint64_t out_bytes = (uint64_t)total * row_bytes;
    for (int s = 0; s < world; ++s)
      if (overlaps((uintptr_t)dst, out_bytes, (uintptr_t)srcs[s], (uint64_t)rows_per_src[s] * row_bytes))
        return PLR_EINVAL;
  }
  a.dst = static_cast<uint8_t*>(dst);
  a.counts = counts;
  a.offsets = offsets;
  const CopyVScratch layout = copy_v_scratch(world, rows_per_src);
  a.ticket = static_cast<uint32_t*>(scratch);
  a.key = reinterpret_cast<uint32_t*>(static_cast<char*>(scratch) + layout.key_off);
  a.seg_count = reinterpret_cast<int32_t*>(static_cast<char*>(scratch) + layout.count_off);
  a.seg_out = reinterpret_cast<int32_t*>(static_cast<char*>(scratch) + layout.out_off);
  a.seg_start[0] = 0;
  for (int s = 0; s < world; ++s)
    a.seg_start[s + 1] = a.seg_start[s] + (uint32_t)((rows_per_src[s] + kRankSeg - 1) / kRankSeg);
  for (int s = world + 1; s <= PLR_MAX_WORLD; ++s) a.seg_start[s] = a.seg_start[world];
  a.row_bytes = row_bytes;
  a.world = (uint32_t)world;
  a.xcd = 0;  // the row scatter runs its workgroups in plain order
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_copy_v(a, s);
  if (e != hipSuccess) return hip_fail(e);
  return PLR_OK;
}

extern "C" int plr_allreduce(plr_layout* L, const void* const* srcs, void* const* dsts,
                             void* workspace, void* stream) {
  if (!L || L->op != PLR_OP_ALLREDUCE || !srcs || !dsts) return PLR_EINVAL;
  const int W = L->world;
  const uint64_t S = L->seg_len;
  for (int w = 0; w < W; ++w) {
    if (!srcs[w] || !dsts[w]) return PLR_EINVAL;
    if (!a16(srcs[w]) || !a16(dsts[w])) return PLR_EALIGN;
  }
  for (int w = 0; w < W; ++w)
    for (int v = 0; v < W; ++v) {
      if (overlaps((uintptr_t)dsts[w], S, (uintptr_t)srcs[v], S)) return PLR_EINVAL;
      if (v != w && overlaps((uintptr_t)dsts[w], S, (uintptr_t)dsts[v], S)) return PLR_EINVAL;
    }
  const bool composed = L->datapath == PLR_PATH_COMPOSED;
  if (composed && !workspace) return PLR_EINVAL;
  if (workspace && !a16(workspace)) return PLR_EALIGN;
  if (!L->ntiles) return PLR_OK;
  AllReduceArgs a{};
  for (int w = 0; w < W; ++w) {
    a.src[w] = static_cast<const u32x4*>(srcs[w]);
    a.dst[w] = static_cast<u32x4*>(dsts[w]);
  }
  a.slice_vecs = S / W / 16;
  a.tile_vecs = L->tile_bytes / 16;
  a.tiles_per_slice = L->tiles_per_seg;
  a.ntiles = L->ntiles;
  a.world = (uint32_t)W;
  a.run = 1;
  a.lag = (uint32_t)L->lag;
  Launch l{};
  l.block = (uint32_t)L->block;
  l.datapath = L->datapath;
  l.lds_bytes = composed ? 0 : L->lds_reserve;
  if (composed) {
    a.nt.err = static_cast<uint64_t*>(workspace);
    a.nt.flags = reinterpret_cast<const uint64_t*>(static_cast<char*>(workspace) + kWorkspaceHeader);
    a.nt.epoch = L->epoch + 1;
    a.nt.spin_limit = L->spin_limit;
    l.grid = L->ntiles + a.lag;
  } else {
    a.run = run_for(L, false);
    l.grid = (uint32_t)std::max<uint64_t>(1, ((uint64_t)L->ntiles + a.run - 1) / a.run);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_allreduce(a, L->dtype, l, s);
  if (e != hipSuccess) return hip_fail(e);
  if (composed) L->epoch = a.nt.epoch;
  return PLR_OK;
}

// Packet buffers hold two slots of 2 x the share each; epoch e uses slot e & 1 (section 4.3
// "Epoch Bookkeeping": the epoch's parity selects one of two staging buffers), so a
// producer may pack epoch e + 1 while the consumer of epoch e still reads its packets.
static uint64_t packet_slot_bytes(const plr_layout* L) { return 2 * L->seg_len; }

extern "C" size_t plr_layout_packet_bytes(const plr_layout* L) {
  return (L && L->op == PLR_OP_REDUCE) ? 2 * (size_t)packet_slot_bytes(L) : 0;
}

extern "C" int plr_pack(plr_layout* L, int src, const void* const* data, void* const* packets,
                        void* stream) {
  if (!L || L->op != PLR_OP_REDUCE || !data || !packets) return PLR_EINVAL;
  if (src < -1 || src >= L->world) return PLR_EINVAL;
  const int s0 = src < 0 ? 0 : src, s1 = src < 0 ? L->world : src + 1;
  PackArgs a{};
  for (int s = s0; s < s1; ++s) {
    if (!data[s] || !packets[s]) return PLR_EINVAL;
    if (!a16(data[s]) || !a16(packets[s])) return PLR_EALIGN;
    const char* share = static_cast<const char*>(data[s]) + L->segs[s].src_off;
    const uint64_t pb = plr_layout_packet_bytes(L);
    for (int t = s0; t < s1; ++t) {  // a packet buffer overlaps no share and no other buffer
      const char* other = static_cast<const char*>(data[t]) + L->segs[t].src_off;
      if (overlaps((uintptr_t)packets[s], pb, (uintptr_t)other, L->seg_len)) return PLR_EINVAL;
      if (t != s && overlaps((uintptr_t)packets[s], pb, (uintptr_t)packets[t], pb)) return PLR_EINVAL;
    }
    a.data[s] = reinterpret_cast<const uint32_t*>(share);
    a.packets[s] = static_cast<uint64_t*>(packets[s]);
  }
  if (!L->seg_len) return PLR_OK;
  const uint64_t epoch = L->epoch + 1;
  for (int s = s0; s < s1; ++s)  // this epoch's slot
    a.packets[s] = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(a.packets[s]) +
                                               (epoch & 1) * packet_slot_bytes(L));
  a.nwords = L->seg_len / 4;
  a.first = (uint32_t)s0;
  a.stamp = (uint32_t)epoch;
  hipError_t e = launch_pack(a, (uint32_t)(s1 - s0), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return PLR_OK;
}

extern "C" int plr_reduce_packets(plr_layout* L, const void* const* packets, void* dst, void* workspace,
                                  void* stream) {
  if (!L || L->op != PLR_OP_REDUCE || !packets || !dst || !workspace) return PLR_EINVAL;
  if (!a16(dst) || !a16(workspace)) return PLR_EALIGN;
  for (int w = 0; w < L->world; ++w) {
    if (!packets[w]) return PLR_EINVAL;
    if (!a16(packets[w])) return PLR_EALIGN;
    if (overlaps((uintptr_t)dst, L->seg_len, (uintptr_t)packets[w], plr_layout_packet_bytes(L))) return PLR_EINVAL;
  }
  const uint64_t epoch = L->epoch + 1;
  if (L->seg_len) {
    PacketReduceArgs a{};
    for (int w = 0; w < L->world; ++w)  // this epoch's slot
      a.pk[w] = reinterpret_cast<const uint64_t*>(static_cast<const char*>(packets[w]) +
                                                  (epoch & 1) * packet_slot_bytes(L));
    a.dst = static_cast<uint32_t*>(dst);
    a.nwords = L->seg_len / 4;
    a.world = (uint32_t)L->world;
    a.stamp = (uint32_t)epoch;
    a.err = static_cast<uint64_t*>(workspace);
    a.spin_limit = L->spin_limit;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_reduce_packets(a, L->dtype, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  L->epoch = epoch;
  return PLR_OK;
}

extern "C" int plr_notify(plr_layout* L, int src, void* workspace, void* stream) {
  if (!L || !workspace) return PLR_EINVAL;
  if (L->op == PLR_OP_ALLREDUCE) return PLR_EINVAL;
  if (src < -1 || src >= L->world) return PLR_EINVAL;
  if (!a16(workspace)) return PLR_EALIGN;
  if (L->nchunks == 0) return PLR_OK;
  NotifyArgs a{};
  uint64_t* flags = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + kWorkspaceHeader);
  if (src < 0) {
    a.flags = flags;
    a.nflags = nflags(L);
  } else {
    uint64_t first, count;
    src_flags(L, src, &first, &count);
    if (count == 0) return PLR_OK;
    a.flags = flags + first;
    a.nflags = count;
  }
  a.epoch = L->epoch + 1;
  hipError_t e = launch_notify(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return PLR_OK;
}

extern "C" int plr_check(plr_layout* L, void* workspace, void* stream) {
  if (!L || !workspace) return PLR_EINVAL;
  if (!a16(workspace)) return PLR_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint64_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  if (v != 0) {
    const uint64_t zero = 0;
    e = hipMemcpyAsync(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e);
    return v == PLR_ETIMEOUT ? PLR_ETIMEOUT : PLR_EINVAL;
  }
  return PLR_OK;
}

extern "C" int plr_set_timing_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr)) return PLR_EINVAL;
  g_timing = Timing{static_cast<hipEvent_t>(before), static_cast<hipEvent_t>(after), nullptr, nullptr};
  return PLR_OK;
}

extern "C" int plr_set_timing_events_split(void* before, void* first_after, void* last_before, void* after) {
  const int set = (before != nullptr) + (first_after != nullptr) + (last_before != nullptr) + (after != nullptr);
  if (set != 0 && set != 4) return PLR_EINVAL;
  g_timing = Timing{static_cast<hipEvent_t>(before), static_cast<hipEvent_t>(after),
                    static_cast<hipEvent_t>(first_after), static_cast<hipEvent_t>(last_before)};
  return PLR_OK;
}

extern "C" const char* plr_strerror(int code) {
  switch (code) {
    case PLR_OK: return "success";
    case PLR_EINVAL: return "invalid argument";
    case PLR_EALIGN: return "address or byte count not a multiple of 16";
    case PLR_EUNSUPPORTED: return "unsupported configuration";
    case PLR_EHIP: return "HIP runtime error";
    case PLR_ETIMEOUT: return "chunk notification timed out";
    case PLR_ETOOLARGE: return "request needs more scratch than the allocation-free entry point holds";
    default: return "unknown error";
  }
}

extern "C" int plr_last_hip_error(void) { return g_last_hip; }

extern "C" const char* plr_version(void) { return "plr 0.1.0 gfx950"; }
