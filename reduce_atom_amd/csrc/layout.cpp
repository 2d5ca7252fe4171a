// Layout compile (host only): a collective specification becomes a segment table, a
// chunk count and a resolved launch policy.
//
// Purlin paper, section 3.1 "Layouts": a collective is a naming of an input and an
// output layout plus copy or reduce; the kinds are packed, scattered and transposed.
// Section 3.2 "SNAC" derives the rank dependencies from the layouts: here that is the
// table saying which (source, offset) feeds which output range. Section 4.2 "Codesign
// Policies and Tuning": chunk sizes, workgroup counts and pipeline depths come from a
// per-GPU table that callers may override.
#include "layout.h"

#include <string.h>

#include <algorithm>
#include <new>

#include "kernels.h"

namespace plr {

size_t elem_bytes(plr_dtype t) { return t == PLR_F32 ? 4 : 2; }

// gfx950 policy table (measured on MI355X with 8 x 117 MB bf16 reduces and 512 MiB
// copies): the best streaming rate comes from short steps per workgroup and a grid
// that covers every tile, so the dispatcher walks the whole chip through memory front
// to back, in plain workgroup order; 16-byte non-temporal loads and stores. Tiles of
// 128 threads: 2 KiB per source for the reduce (one vector per lane per source), one
// per workgroup; 4 KiB for copies of over 2 MiB from some source, one per workgroup, else
// 2 KiB, two per workgroup once a call has 4096 tiles (8 MiB) or more. Flags cover 256 KiB
// chunks (16 KiB for decode-size shares). With in-kernel waits a notified workgroup pays
// one agent-scope acquire per chunk it enters, and those acquires invalidate L2 lines, so
// such calls give each workgroup a run of 2 (reduce) or 4 (copy) tiles; decode-size reduce
// shares (at most 2 MiB per source) keep one tile per workgroup, where latency rules: 4 KiB
// tiles of 256 threads, and for notified calls over 512 KiB per source 8 KiB of 512.
constexpr uint64_t kCus = 256;  // compute units of an MI355X (the composed AllReduce's tiles)
constexpr uint32_t kLdsPerCu = 160u << 10;  // LDS bytes per compute unit of gfx950

static void default_policy(plr_layout* L) {
  L->stages = 0;  // no ring on the direct path
  L->datapath = PLR_PATH_DIRECT;
  L->workgroups = 0;
  L->run = 1;  // one tile per workgroup (copies: set from the tile count below)
  // XCD-contiguous order cost the reduce 1-8% and the copies at their policy run 0-7%
  L->xcd_order = kXcdOff;
  // throughput regime: check first, so that stream-ordered producers cost no per-chunk
  // acquires; latency regime (at most 2 MiB from any source): wait inside the kernel (a
  // check launch costs more). Judged by the bytes per source, not per segment: a
  // notified AllToAll of 8 x 4 MiB (512 KiB slices) took 42.5 us with in-kernel waits.
  L->notify_mode = L->src_bytes <= (2u << 20) ? PLR_NOTIFY_CHUNKS : PLR_NOTIFY_CHECK;
  L->run_notified = L->op == PLR_OP_REDUCE ? 2 : 4;
  if (L->op == PLR_OP_REDUCE) {
    if (L->src_bytes <= (2u << 20)) {  // latency regime: every tile in one dispatch wave
      // 4 KiB tiles of 256 threads; over 512 KiB per source, notified calls take 8 KiB
      // tiles of 512 threads (16 KiB chunks either way) and un-notified ones keep 4 KiB
      // of 256 (set after the tables below). Measured per call (notify + reduce, replayed
      // graph) on 8 x [T, 7168] bf16: T = 64, 5.84 us against 6.67 us for 4 KiB tiles;
      // T = 8 slower with 8 KiB
      const bool big = L->src_bytes > (512u << 10);
      L->block = big ? 512 : 256;
      L->unroll = 1;
      L->tile_bytes = big ? 8u << 10 : 4u << 10;
      L->chunk_bytes = 16u << 10;
      L->run_notified = 1;
    } else {
      L->block = 128;
      L->unroll = 1;
      L->tile_bytes = 2u << 10;
      L->chunk_bytes = 256u << 10;
    }
  } else if (L->op == PLR_OP_COPY) {
    // throughput regime (over 2 MiB from a source): 4 KiB tiles, one per workgroup (each
    // lane moves two vectors in turn); measured on 8 x 64 MiB, AllGather 158-159 us and AllToAll 159 us against
    // 165 us for 2 KiB tiles in runs of 2, notified or not, while 4 KiB at 256 threads
    // took 187 us, 8 KiB 166-170 us and 16 KiB 173-176 us
    L->block = 128;
    L->unroll = 1;
    L->tile_bytes = L->src_bytes > (2u << 20) ? 4u << 10 : 2u << 10;
    L->chunk_bytes = 256u << 10;
  } else {  // allreduce: fused by default; the composed path's tiles follow the slice
    L->block = 128;
    L->unroll = 1;
    L->tile_bytes = 2u << 10;
    L->chunk_bytes = L->tile_bytes;
  }
  // composed AllReduce: workgroup b gathers the tile of workgroup b - lag. The
  // dispatcher hands workgroup b to XCD b % 8 and dispatches each XCD's workgroups in
  // increasing order, so with a multiple of 8 the producer sits on the same XCD and
  // was dispatched first: every wait is for a resident or finished workgroup.
  L->lag = 16;
}

}  // namespace plr

using namespace plr;

static bool aligned16(uint64_t x) { return (x & 15) == 0; }

extern "C" int plr_layout_create(const plr_layout_desc* d, plr_layout** out) {
  if (!d || !out) return PLR_EINVAL;
  *out = nullptr;
  // A C caller may store any int in the enum-typed fields, and loading a value outside
  // an enumeration's range through its type is undefined in C++: read them as ints.
  static_assert(sizeof(plr_op) == sizeof(int) && sizeof(plr_dtype) == sizeof(int) &&
                    sizeof(plr_layout_kind) == sizeof(int),
                "the descriptor's enum fields are ints");
  auto field = [](const void* p) {
    int v;
    memcpy(&v, p, sizeof v);
    return v;
  };
  const int op = field(&d->op), dtype = field(&d->dtype);
  const int in_kind = field(&d->in_kind), out_kind = field(&d->out_kind);
  if (d->world < 1) return PLR_EINVAL;
  if (d->world > PLR_MAX_WORLD) return PLR_EUNSUPPORTED;
  if (d->mode != PLR_MODE_DETERMINISTIC) return PLR_EUNSUPPORTED;
  if (op != PLR_OP_REDUCE && op != PLR_OP_COPY && op != PLR_OP_ALLREDUCE) return PLR_EINVAL;
  if (dtype != PLR_BF16 && dtype != PLR_F16 && dtype != PLR_F32) return PLR_EINVAL;
  if (in_kind < PLR_PACKED || in_kind > PLR_TRANSPOSED) return PLR_EINVAL;
  if (out_kind < PLR_PACKED || out_kind > PLR_TRANSPOSED) return PLR_EINVAL;
  if (!aligned16(d->bytes_per_src)) return PLR_EALIGN;

  plr_layout* L = new (std::nothrow) plr_layout();
  if (!L) return PLR_EINVAL;
  L->op = (plr_op)op;
  L->dtype = (plr_dtype)dtype;
  L->world = d->world;
  L->rank = d->rank;
  L->bytes_per_src = d->bytes_per_src;
  L->in_kind = (plr_layout_kind)in_kind;
  L->out_kind = (plr_layout_kind)out_kind;
  L->epoch = 0;

  const int W = d->world;
  const uint64_t B = d->bytes_per_src;
  auto fail = [&](int code) {
    delete L;
    return code;
  };

  // variable-length partitions: sizes and their exclusive prefix sums
  const bool var = d->part_bytes != nullptr;
  std::vector<uint64_t> part(W, 0), part0(W + 1, 0);
  if (var) {
    if (op == PLR_OP_ALLREDUCE) return fail(PLR_EINVAL);
    for (int w = 0; w < W; ++w) {
      part[w] = d->part_bytes[w];
      if (!aligned16(part[w])) return fail(PLR_EALIGN);
      if (part[w] > B - part0[w]) return fail(PLR_EINVAL);  // past T (and no wrapped sum)
      part0[w + 1] = part0[w] + part[w];
    }
    if (part0[W] != B) return fail(PLR_EINVAL);  // the sizes add up to the message size T
  }
  L->var_segs = false;

  if (op == PLR_OP_REDUCE) {
    if (out_kind != PLR_PACKED || d->out_offsets) return fail(PLR_EINVAL);
    uint64_t share, off;
    if (in_kind == PLR_PACKED) {
      if (var) return fail(PLR_EINVAL);  // partitions only make sense for a scattered input
      share = B;
      off = 0;
    } else if (in_kind == PLR_SCATTERED) {
      if (d->rank < 0 || d->rank >= W) return fail(PLR_EINVAL);
      if (var) {  // ReduceScatterV: partition `rank` of every source
        share = part[d->rank];
        off = part0[d->rank];
      } else {
        if (B % (16ull * W)) return fail(PLR_EALIGN);
        share = B / W;
        off = (uint64_t)d->rank * share;
      }
    } else {
      return fail(PLR_EINVAL);
    }
    for (int w = 0; w < W; ++w) {
      const uint64_t o = d->in_offsets ? d->in_offsets[w] : off;
      if (!aligned16(o)) return fail(PLR_EALIGN);
      if (o > ~0ull - share) return fail(PLR_EINVAL);  // the share's end would wrap around
      L->segs.push_back({w, o, 0, share});
    }
    L->seg_len = share;
    L->dst_bytes = share;
  } else if (op == PLR_OP_ALLREDUCE) {
    if (in_kind != PLR_SCATTERED || out_kind != PLR_SCATTERED) return fail(PLR_EINVAL);
    if (d->in_offsets || d->out_offsets) return fail(PLR_EINVAL);
    if (B % (16ull * W)) return fail(PLR_EALIGN);
    for (int w = 0; w < W; ++w) L->segs.push_back({w, 0, 0, B});
    L->seg_len = B;
    L->dst_bytes = B;
  } else {
    if (in_kind == PLR_PACKED && out_kind == PLR_PACKED && var) {  // AllGatherV
      uint64_t longest = 0;
      for (int s = 0; s < W; ++s) {
        L->segs.push_back({s, 0, part0[s], part[s]});
        longest = std::max(longest, part[s]);
      }
      L->seg_len = longest;
      L->var_segs = true;
    } else if (var) {
      return fail(PLR_EINVAL);  // the other copies have no variable-length form here
    } else if (in_kind == PLR_PACKED && out_kind == PLR_PACKED) {  // AllGather
      for (int s = 0; s < W; ++s) L->segs.push_back({s, 0, (uint64_t)s * B, B});
      L->seg_len = B;
    } else if (in_kind == PLR_SCATTERED &&
               (out_kind == PLR_TRANSPOSED || out_kind == PLR_SCATTERED)) {
      if (B % (16ull * W)) return fail(PLR_EALIGN);
      const uint64_t t = B / W;
      if (out_kind == PLR_TRANSPOSED) {  // AllToAll: out slice (d, s) = in slice (s, d)
        for (int s = 0; s < W; ++s)
          for (int dd = 0; dd < W; ++dd)
            L->segs.push_back({s, (uint64_t)dd * t, ((uint64_t)dd * W + s) * t, t});
      } else {  // gather half of AllReduce: out slice s = slice s of source s
        for (int s = 0; s < W; ++s) L->segs.push_back({s, (uint64_t)s * t, (uint64_t)s * t, t});
      }
      L->seg_len = t;
    } else {
      return fail(PLR_EINVAL);
    }
    const size_t nseg = L->segs.size();
    if ((d->in_offsets || d->out_offsets) && nseg > (size_t)kMaxTableSegs)
      return fail(PLR_EUNSUPPORTED);
    for (size_t k = 0; k < nseg; ++k) {
      if (d->in_offsets) L->segs[k].src_off = d->in_offsets[k];
      if (d->out_offsets) L->segs[k].dst_off = d->out_offsets[k];
      if (!aligned16(L->segs[k].src_off) || !aligned16(L->segs[k].dst_off)) return fail(PLR_EALIGN);
      const uint64_t len = L->segs[k].len;  // no segment end may wrap around
      if (L->segs[k].src_off > ~0ull - len || L->segs[k].dst_off > ~0ull - len) return fail(PLR_EINVAL);
    }
    // output segments must not overlap (two writers of one byte would race)
    std::vector<std::pair<uint64_t, uint64_t>> iv;
    for (auto& s : L->segs)
      if (s.len) iv.push_back({s.dst_off, s.dst_off + s.len});
    std::sort(iv.begin(), iv.end());
    L->dst_bytes = 0;
    for (size_t k = 0; k < iv.size(); ++k) {
      if (k && iv[k].first < iv[k - 1].second) return fail(PLR_EINVAL);
      L->dst_bytes = std::max<uint64_t>(L->dst_bytes, iv[k].second);
    }
    L->table_fits = nseg <= (size_t)kMaxTableSegs;
  }

  // policy: built-in table, then the caller's overrides
  {
    std::vector<uint64_t> per(W, 0);
    for (auto& s : L->segs) per[s.src] += s.len;
    L->src_bytes = 0;
    for (uint64_t v : per) L->src_bytes = std::max(L->src_bytes, v);
  }
  default_policy(L);
  if (d->tile_bytes) {
    if (!aligned16(d->tile_bytes)) return fail(PLR_EALIGN);
    L->tile_bytes = d->tile_bytes;
  }
  if (d->chunk_bytes) {
    if (!aligned16(d->chunk_bytes)) return fail(PLR_EALIGN);
    L->chunk_bytes = d->chunk_bytes;
    if (!d->tile_bytes) L->tile_bytes = std::min<uint64_t>(L->tile_bytes, L->chunk_bytes);
  }
  if (d->workgroups < 0) return fail(PLR_EINVAL);
  if (d->workgroups) L->workgroups = d->workgroups;
  if (d->block) {
    if (d->block != 64 && d->block != 128 && d->block != 256 && d->block != 512) return fail(PLR_EINVAL);
    L->block = d->block;
  }
  if (d->unroll) {
    if (d->unroll != 1 && d->unroll != 2 && d->unroll != 4) return fail(PLR_EINVAL);
    L->unroll = d->unroll;
  }
  // a reduce lane holds unroll x W vectors at once: 4 x 15 or 4 x 16 no longer fit the
  // registers (the compiler spills them), so those take 2 vectors per lane
  if (L->op == PLR_OP_REDUCE && L->unroll * W > 56) L->unroll = 2;
  if (d->stages) {
    if (d->stages < 1 || d->stages > 4) return fail(PLR_EINVAL);
    L->stages = d->stages;
  }
  if (d->datapath) {
    if (d->datapath != PLR_PATH_DIRECT && d->datapath != PLR_PATH_LDS && d->datapath != PLR_PATH_COMPOSED)
      return fail(PLR_EINVAL);
    if ((d->datapath == PLR_PATH_COMPOSED) != (op == PLR_OP_ALLREDUCE && d->datapath != PLR_PATH_DIRECT))
      return fail(PLR_EINVAL);  // composed is the AllReduce role split; AllReduce has no LDS path
    L->datapath = d->datapath;
    if (d->datapath == PLR_PATH_COMPOSED) {
      if (!d->tile_bytes) L->tile_bytes = 0;  // chosen from the slice below
      if (!d->block) L->block = 256;
    }
  }
  if (L->var_segs && L->datapath == PLR_PATH_LDS) return fail(PLR_EUNSUPPORTED);
  // resident workgroups per CU, capped through an LDS reservation at launch. The fused
  // AllReduce of more than 2 MiB per source keeps 8: graph replays of 8 sources into 8
  // outputs, against uncapped on one machine, ran 1-4% faster at every placement tried (64 MiB
  // per source 64 MiB, 1 GiB + 2 MiB or 2 GiB apart 184-190 us against 188-192 us; in the
  // collective sweep's 1 GiB buffers 191.8 against 193.6 us; [8192, 7168] bf16 in separate
  // tensors 326-327 against 334 us) and was never more than 0.4% slower (512 MiB apart: 193.0
  // against 192.3 us). Fewer workgroups gain more where the 16 streams per tile fall on
  // different places of the HBM address map (3 per CU: 164-172 us at 64 MiB or 1 GiB + 2 MiB
  // apart, 308 us for the separate tensors) but lose 10-25% where their start addresses
  // collide there (the pattern an XOR of address bits that includes the high ones would
  // give; no rule on the addresses predicted it): 233-239 us at 512 MiB or 2 GiB apart,
  // 257-260 us at 1 GiB + 4 MiB against 212 us, 214-217 us in the sweep's buffers. So 3 stays
  // the caller's choice. Every other kernel is slower capped: the 8 x 117 MB reduce took
  // 162.2-163.3 us uncapped, the same at 6 or 8 per CU and 174-177 us at 4 or 5; the 512 MiB
  // copy gained nothing that held; the AllToAllV row scatter, which lives on many short
  // workgroups, 150 us uncapped against 155-440 us at 11 down to 2 per CU.
  if (d->wgs_per_cu < -1 || d->wgs_per_cu > 16)
    return fail(PLR_EINVAL);
  if (d->wgs_per_cu > 0)
    L->wgs_per_cu = d->wgs_per_cu;
  else if (d->wgs_per_cu == 0)
    L->wgs_per_cu = op == PLR_OP_ALLREDUCE && L->src_bytes > (2u << 20) ? 8 : 0;
  else
    L->wgs_per_cu = 0;
  if (L->datapath != PLR_PATH_DIRECT) L->wgs_per_cu = 0;  // LDS-staged and composed: never capped
  // the reservation leaves 512 bytes of each share for the kernel's own workgroup memory
  // (the direct reduce and copy use 256 bytes, for the workgroup-wide vote of their chunk
  // waits), so that exactly wgs_per_cu workgroups fit
  L->lds_reserve = L->wgs_per_cu ? ((kLdsPerCu / (uint32_t)L->wgs_per_cu) - 512u) & ~511u : 0;
  if (L->datapath == PLR_PATH_LDS) {
    // the staged pipeline runs 256-thread workgroups over 4 KiB slabs per source. Measured
    // on the 8 x 117 MB reduce and the 8 x 64 MiB AllGather (ring depth x slabs per
    // workgroup): the reduce is fastest with 2 stages and one slab per workgroup (two
    // workgroups per CU by their 64 KiB of LDS), 170.6-171.7 us against 177-180 us at 2
    // slabs, 184-186 us for the earlier 3 stages x 4 slabs and 165-166 us on the
    // register-staged path; one stage (32 KiB: 3 to 5 workgroups per CU) took 175-187 us.
    // The copy is fastest with 4 stages and 2 slabs per workgroup, 165-169 us against
    // 178-182 us for the earlier 8 stages x 8 slabs and 159-160 us register-staged; fewer
    // workgroups per CU (LDS padded to 2-5 per CU) took 200-300 us
    if (d->block && d->block != 256) return fail(PLR_EINVAL);
    L->block = 256;
    if (!d->tile_bytes && L->tile_bytes % 4096) L->tile_bytes = 4096;
    L->stages = op == PLR_OP_REDUCE ? lds_reduce_stages(W) : kCopyStages;
    const int slabs = op == PLR_OP_REDUCE ? (W <= 4 ? L->stages + 1 : 1) : 2;
    const uint64_t per_tile = L->tile_bytes / 4096 ? L->tile_bytes / 4096 : 1;
    L->run = L->run_notified = (int)std::max<uint64_t>(1, (uint64_t)slabs / per_tile);
  }
  L->spin_limit = d->spin_limit ? d->spin_limit : kDefaultSpinLimit;
  if (d->xcd_order) {
    if (d->xcd_order != 1 && d->xcd_order != 2) return fail(PLR_EINVAL);
    L->xcd_order = d->xcd_order == 1 ? kXcdOn : kXcdOff;
  }
  if (d->notify_mode) {
    if (d->notify_mode != PLR_NOTIFY_CHUNKS && d->notify_mode != PLR_NOTIFY_CHECK) return fail(PLR_EINVAL);
    L->notify_mode = d->notify_mode;
  }
  // in check mode only chunks still missing at check time pay a wait and a fence, so
  // notified calls can use shorter runs (measured: reduce 1, copy 2 tiles of 2 KiB or 1
  // of 4 KiB)
  if (L->notify_mode == PLR_NOTIFY_CHECK && L->datapath != PLR_PATH_LDS)
    L->run_notified = L->op == PLR_OP_REDUCE || L->tile_bytes >= 4096 ? 1 : 2;

  // tile and chunk tables; a chunk is a whole number of tiles of one segment
  if (L->op == PLR_OP_ALLREDUCE) {  // tiles of the W slices; one flag per tile
    const uint64_t slice = L->seg_len / W;
    if (slice == 0) {
      L->tiles_per_seg = L->tiles_per_chunk = L->chunks_per_seg = 0;
      L->ntiles = L->nchunks = 0;
    } else {
      uint64_t tile = L->tile_bytes;
      if (tile == 0) {
        // composed policy: every tile pays one agent-scope release, an L2 writeback
        // that the XCD's workgroups go through one at a time, so take as few tiles as
        // keep every CU busy with all ntiles + lag workgroups resident in one round;
        // whole steps of the workgroup (block x 16 bytes) when a tile holds one
        const uint64_t per_slice = std::max<uint64_t>(1, (kCus - L->lag) / (uint64_t)W);
        const uint64_t raw = (slice + per_slice - 1) / per_slice;
        const uint64_t step = (uint64_t)L->block * 16;
        const uint64_t g = raw >= step ? step : 16;
        tile = (raw + g - 1) / g * g;
      }
      tile = std::min<uint64_t>(tile, slice);
      const uint64_t tps = (slice + tile - 1) / tile;
      if (tps * W > 0x7FFFFFFFull) return fail(PLR_EUNSUPPORTED);
      L->tile_bytes = L->chunk_bytes = tile;
      L->tiles_per_seg = (uint32_t)tps;  // tiles per slice
      L->tiles_per_chunk = L->chunks_per_seg = 1;
      L->ntiles = L->nchunks = (uint32_t)(tps * W);
      // The composed kernel's gatherers wait for reducers of lower workgroup ids; with
      // every workgroup of the call resident at once (one per CU at most) each waited-for
      // reducer is running, whatever order the workgroups are dispatched in. A caller's
      // tile size that needs more workgroups than that is refused.
      if (L->datapath == PLR_PATH_COMPOSED && (uint64_t)L->ntiles + (uint64_t)L->lag > kCus)
        return fail(PLR_EUNSUPPORTED);
    }
  } else if (L->seg_len == 0) {
    L->tiles_per_seg = L->tiles_per_chunk = L->chunks_per_seg = 0;
    L->ntiles = L->nchunks = 0;
  } else {
    const uint64_t tile = std::min<uint64_t>(L->tile_bytes, L->seg_len);
    const uint64_t tps = (L->seg_len + tile - 1) / tile;  // of the longest segment
    uint64_t tpc = std::max<uint64_t>(1, (L->chunk_bytes + tile - 1) / tile);
    tpc = std::min<uint64_t>(tpc, tps);
    const uint64_t cps = (tps + tpc - 1) / tpc;
    const uint64_t nseg = L->op == PLR_OP_REDUCE ? 1 : L->segs.size();
    if (tps * nseg > 0x7FFFFFFFull) return fail(PLR_EUNSUPPORTED);
    if (L->datapath == PLR_PATH_LDS && tps > 1 && tile % 4096) return fail(PLR_EINVAL);
    L->tile_bytes = tile;
    L->chunk_bytes = tile * tpc;
    L->tiles_per_seg = (uint32_t)tps;
    L->tiles_per_chunk = (uint32_t)tpc;
    L->chunks_per_seg = (uint32_t)cps;
    L->ntiles = (uint32_t)(tps * nseg);
    L->nchunks = (uint32_t)(cps * nseg);
    if (L->var_segs) {  // every segment its own tile and chunk count
      // Partition sizes are multiples of 16 bytes only, so a segment's destination may
      // start inside a 128-byte line: its tiles are then cut on the destination's lines
      // (tile 0 short by the offset into the line), or every store would write partial
      // lines at both ends, which neighbouring workgroups share (measured on the 1 GiB
      // AllGatherV: 337-340 us with 16-byte offsets, 323 us with line-aligned ones).
      // Chunks keep their byte ranges; a shifted tile may span two of them.
      uint64_t tiles = 0, chunks = 0;
      for (uint64_t k = 0; k < nseg; ++k) {
        L->seg_tile0.push_back((uint32_t)tiles);
        L->seg_chunk0.push_back((uint32_t)chunks);
        const uint64_t len = L->segs[k].len;
        const uint32_t sh = tile >= 256 ? (uint32_t)(L->segs[k].dst_off % 128) : 0;
        L->seg_shift.push_back(sh);
        tiles += len ? (len + sh + tile - 1) / tile : 0;
        chunks += ((len + tile - 1) / tile + tpc - 1) / tpc;
      }
      L->seg_tile0.push_back((uint32_t)tiles);
      L->seg_chunk0.push_back((uint32_t)chunks);
      L->ntiles = (uint32_t)tiles;
      L->nchunks = (uint32_t)chunks;
    }
  }
  // copies of 2 KiB tiles: runs of 2 once a call has 4096 tiles, as in check mode
  // (measured without notification on 8 sources: AllGather and AllToAll of 8 x 64 MiB
  // 166 us with runs of 2 against 184-189 us with 1, AllGatherV of 1 GiB 350 against
  // 382 us; at 256 KiB per source one tile per workgroup is as fast or faster)
  if (L->op == PLR_OP_COPY && L->datapath != PLR_PATH_LDS)
    L->run = L->ntiles >= 4096 && L->tile_bytes < 4096 ? 2 : 1;
  if (L->op == PLR_OP_COPY) {  // first flag of every source (segments go source by source)
    const size_t nseg = L->segs.size();
    L->src_flag0.assign(W + 1, 0);
    for (size_t k = 0; k < nseg; ++k) {
      const uint32_t c1 = L->nchunks == 0 ? 0
                          : L->var_segs ? L->seg_chunk0[k + 1]
                                        : (uint32_t)((k + 1) * L->chunks_per_seg);
      L->src_flag0[L->segs[k].src + 1] = c1;
    }
    for (int s = 1; s <= W; ++s) L->src_flag0[s] = std::max(L->src_flag0[s], L->src_flag0[s - 1]);
  }
  L->plain_tile_bytes = L->tile_bytes;
  L->plain_ntiles = L->ntiles;
  L->plain_block = L->block;
  // un-notified reduces of the latency regime keep 4 KiB tiles of 256 threads unless the
  // caller chose a shape. Kernel trace, warm, 8 x [T, 7168] bf16 on one machine: T = 32 /
  // 64 / 128 took 3.04 / 3.72 / 4.64 us against 3.36 / 4.24 / 4.72 us with 8 KiB tiles of
  // 512 threads, which the notified calls keep (4.68 / 5.84 / 7.04 against 4.76 / 6.00 /
  // 8.36 us with 4 KiB tiles)
  if (L->op == PLR_OP_REDUCE && L->datapath == PLR_PATH_DIRECT && L->src_bytes <= (2u << 20) &&
      L->seg_len && !d->tile_bytes && !d->chunk_bytes && !d->block) {
    const uint64_t t = std::min<uint64_t>(4u << 10, L->seg_len);
    L->plain_tile_bytes = t;
    L->plain_ntiles = (uint32_t)((L->seg_len + t - 1) / t);
    L->plain_block = 256;
  }
  *out = L;
  return PLR_OK;
}

extern "C" void plr_layout_destroy(plr_layout* L) { delete L; }

extern "C" size_t plr_layout_workspace_bytes(const plr_layout* L) {
  if (!L) return 0;
  if (L->op == PLR_OP_ALLREDUCE) return kWorkspaceHeader + (size_t)L->nchunks * sizeof(uint64_t);
  return kWorkspaceHeader + 2 * (size_t)nflags(L) * sizeof(uint64_t);
}

extern "C" size_t plr_layout_dst_bytes(const plr_layout* L) { return L ? L->dst_bytes : 0; }
extern "C" int plr_layout_nchunks(const plr_layout* L) { return L ? (int)L->nchunks : -1; }
extern "C" int plr_layout_ntiles(const plr_layout* L) { return L ? (int)L->ntiles : -1; }
extern "C" int plr_layout_nsegments(const plr_layout* L) { return L ? (int)L->segs.size() : -1; }
extern "C" uint64_t plr_layout_epoch(const plr_layout* L) { return L ? L->epoch : 0; }

extern "C" int plr_layout_segment(const plr_layout* L, int k, int* src, size_t* src_off,
                                  size_t* dst_off, size_t* len) {
  if (!L || k < 0 || k >= (int)L->segs.size()) return PLR_EINVAL;
  const auto& s = L->segs[k];
  if (src) *src = s.src;
  if (src_off) *src_off = s.src_off;
  if (dst_off) *dst_off = s.dst_off;
  if (len) *len = s.len;
  return PLR_OK;
}

extern "C" int plr_layout_policy(const plr_layout* L, size_t* tile_bytes, size_t* chunk_bytes,
                                 int* workgroups, int* block, int* unroll, int* stages,
                                 int* datapath, int* notify_mode) {
  if (!L) return PLR_EINVAL;
  if (tile_bytes) *tile_bytes = L->tile_bytes;
  if (chunk_bytes) *chunk_bytes = L->chunk_bytes;
  if (workgroups) *workgroups = L->workgroups;
  if (block) *block = L->block;
  if (unroll) *unroll = L->unroll;
  if (stages) *stages = L->stages;
  if (datapath) *datapath = L->datapath;
  if (notify_mode) *notify_mode = L->notify_mode;
  return PLR_OK;
}

extern "C" int plr_layout_occupancy(const plr_layout* L, int* wgs_per_cu, size_t* lds_bytes) {
  if (!L) return PLR_EINVAL;
  if (wgs_per_cu) *wgs_per_cu = L->wgs_per_cu;
  if (lds_bytes) *lds_bytes = L->lds_reserve;
  return PLR_OK;
}

extern "C" int plr_layout_plain_shape(const plr_layout* L, size_t* tile_bytes, int* block,
                                      int* ntiles) {
  if (!L) return PLR_EINVAL;
  if (tile_bytes) *tile_bytes = L->plain_tile_bytes;
  if (block) *block = L->plain_block;
  if (ntiles) *ntiles = (int)L->plain_ntiles;
  return PLR_OK;
}
