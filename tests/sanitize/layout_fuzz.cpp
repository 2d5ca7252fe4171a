// Host-only fuzz driver for the layout compiler (reduce_atom_amd/csrc/layout.cpp),
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitize.py. It creates layouts from seeded random descriptors,
// valid and invalid, and for every one the compiler accepts checks what the header
// promises: segments inside their source and inside the output, copy segments that
// do not overlap in the output, a resolved policy in range, and accessors that
// answer out-of-range queries with an error.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "plr.h"

static uint64_t g_state;
static uint64_t next_u64() {  // SplitMix64 (Steele, Lea and Flood, 2014)
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static uint64_t below(uint64_t n) { return n ? next_u64() % n : 0; }
template <class T, size_t N>
static T pick(const T (&v)[N]) { return v[below(N)]; }

static const plr_layout_desc* g_desc;  // the descriptor under test, printed on a failure
static void dump() {
  if (!g_desc) return;
  const plr_layout_desc& d = *g_desc;
  int op, dtype, ik, ok;
  memcpy(&op, &d.op, 4), memcpy(&dtype, &d.dtype, 4), memcpy(&ik, &d.in_kind, 4), memcpy(&ok, &d.out_kind, 4);
  fprintf(stderr,
          "  op %d dtype %d world %d rank %d bytes %zu kinds %d->%d in_off %d out_off %d parts %d mode %d "
          "tile %zu chunk %zu workgroups %d block %d unroll %d stages %d datapath %d notify %d xcd %d\n",
          op, dtype, d.world, d.rank, d.bytes_per_src, ik, ok, !!d.in_offsets, !!d.out_offsets, !!d.part_bytes,
          d.mode, d.tile_bytes, d.chunk_bytes, d.workgroups, d.block, d.unroll, d.stages, d.datapath,
          d.notify_mode, d.xcd_order);
}

#define CHECK(c, ...)                                               \
  do {                                                              \
    if (!(c)) {                                                     \
      fprintf(stderr, "iteration %d: check failed: %s: ", it, #c);  \
      fprintf(stderr, __VA_ARGS__);                                 \
      fprintf(stderr, "\n");                                        \
      dump();                                                       \
      abort();                                                      \
    }                                                               \
  } while (0)

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 20000;
  g_state = argc > 2 ? strtoull(argv[2], nullptr, 10) : 1;
  int accepted = 0;
  for (int it = 0; it < iters; ++it) {
    plr_layout_desc d;
    memset(&d, 0, sizeof d);
    // a valid collective most of the time, then policy overrides and mutations
    const int W = (int)pick((const int[]){1, 2, 3, 4, 5, 8, 8, 16});
    const size_t q = 16 * (size_t)W;
    std::vector<size_t> in_off(256), out_off(256), parts(17);
    for (auto& v : in_off) v = 16 * below(1 << 12);
    for (auto& v : out_off) v = 16 * below(1 << 14);
    const int kind = (int)below(8);
    const int ops[8] = {0, 0, 1, 1, 1, 2, 1, 0};      // reduce, reduce, AG, A2A, gather, AR, AGV, RSV
    const int ins[8] = {0, 1, 0, 1, 1, 1, 0, 1};
    const int outs_[8] = {0, 0, 0, 2, 1, 1, 0, 0};
    d.op = (plr_op)ops[kind];
    d.dtype = (plr_dtype)below(3);
    d.world = W;
    d.rank = (int)below((uint64_t)W);
    d.in_kind = (plr_layout_kind)ins[kind];
    d.out_kind = (plr_layout_kind)outs_[kind];
    d.bytes_per_src = pick((const size_t[]){0, q, q * (1 + below(64)), q * (1 + below(1 << 14)),
                                            q * (1 + below(1 << 20)), q << 20});
    if (kind >= 6) {  // variable partitions summing to bytes_per_src
      size_t left = d.bytes_per_src / 16;
      for (int w = 0; w < W; ++w) {
        const size_t take = w + 1 == W ? left : below(left + 1);
        parts[w] = 16 * take;
        left -= take;
      }
      d.part_bytes = parts.data();
    }
    if (kind == 5) d.datapath = (int)pick((const int[]){0, 1, 3});
    if (below(2)) {  // valid policy overrides
      d.tile_bytes = pick((const size_t[]){0, 16, 1024, 2048, 4096, 65536, 16 * (1 + below(4096))});
      d.chunk_bytes = pick((const size_t[]){0, 16, 4096, 65536, 1 << 20});
      d.workgroups = (int)pick((const int[]){0, 1, 3, 1000});
      d.block = (int)pick((const int[]){0, 64, 128, 256, 512});
      d.unroll = (int)pick((const int[]){0, 1, 2, 4});
      d.notify_mode = (int)below(3);
      d.xcd_order = (int)below(3);
      d.wgs_per_cu = (int)pick((const int[]){0, 0, -1, 1, 2, 3, 5, 16});
      if (kind <= 4 && below(3) == 0) d.datapath = 2;  // the LDS path
    }
    if (below(5) == 0) d.in_offsets = in_off.data();
    if (below(5) == 0) d.out_offsets = out_off.data();
    for (int m = (int)below(3) - 1; m > 0 || (m == 0 && below(2)); --m) {  // mutations
      switch (below(19)) {
        case 0: { int v = (int)pick((const int[]){3, -1, 7}); memcpy(&d.op, &v, 4); break; }
        case 1: { int v = (int)pick((const int[]){3, -1}); memcpy(&d.dtype, &v, 4); break; }
        case 2: d.world = (int)pick((const int[]){0, 17, -3}); break;
        case 3: d.rank = (int)pick((const int[]){-1, W, 99}); break;
        case 4: d.bytes_per_src += pick((const size_t[]){8, 16, 24}); break;
        case 5: { int v = (int)below(5) - 1; memcpy(&d.in_kind, &v, 4); break; }
        case 6: { int v = (int)below(5) - 1; memcpy(&d.out_kind, &v, 4); break; }
        case 7: in_off[below(256)] += 8; d.in_offsets = in_off.data(); break;
        case 8: out_off[below(W)] = out_off[0]; d.out_offsets = out_off.data(); break;
        case 9: d.mode = 1; break;
        case 10: d.tile_bytes = pick((const size_t[]){24, 8}); break;
        case 11: d.chunk_bytes = 40; break;
        case 12: d.block = (int)pick((const int[]){1024, 100, 32}); break;
        case 13: d.unroll = 3; d.stages = 5; break;
        case 14: d.datapath = (int)pick((const int[]){4, 2, 3}); d.notify_mode = 3; break;
        case 15: parts[below(W)] += pick((const size_t[]){8, 16}); d.part_bytes = parts.data(); break;
        case 16: in_off[below(W)] = ~(size_t)15 - 16 * below(4); d.in_offsets = in_off.data(); break;
        case 17: d.wgs_per_cu = (int)pick((const int[]){17, -2, 1000}); break;
        default: out_off[below(W)] = ~(size_t)15 - 16 * below(4); d.out_offsets = out_off.data(); break;
      }
    }

    g_desc = &d;
    plr_layout* L = nullptr;
    const int rc = plr_layout_create(&d, &L);
    if (rc != PLR_OK) {
      CHECK(rc == PLR_EINVAL || rc == PLR_EALIGN || rc == PLR_EUNSUPPORTED, "unexpected code %d", rc);
      continue;
    }
    ++accepted;
    CHECK(L != nullptr, "no layout");
    const size_t dst_bytes = plr_layout_dst_bytes(L);
    const int nseg = plr_layout_nsegments(L), ntiles = plr_layout_ntiles(L), nchunks = plr_layout_nchunks(L);
    CHECK(nseg >= 0 && ntiles >= 0 && nchunks >= 0 && nchunks <= std::max(ntiles, 0) + nseg,
          "nseg %d ntiles %d nchunks %d", nseg, ntiles, nchunks);
    CHECK(plr_layout_workspace_bytes(L) >= 256, "workspace %zu", plr_layout_workspace_bytes(L));
    CHECK(plr_layout_epoch(L) == 0, "epoch");
    {  // a capped layout reserves exactly what lets that many workgroups share 160 KiB of LDS
      int cap = -1;
      size_t lds = 1;
      CHECK(plr_layout_occupancy(L, &cap, &lds) == PLR_OK, "occupancy");
      CHECK((cap == 0) == (lds == 0) && cap >= 0 && cap <= 16, "cap %d lds %zu", cap, lds);
      const size_t share = (lds + 256 + 511) / 512 * 512;  // with 256 bytes of the kernel's own
      CHECK(cap == 0 || (int)(163840 / share) == cap, "cap %d lds %zu", cap, lds);
    }
    std::vector<std::pair<size_t, size_t>> outs;
    for (int k = 0; k < nseg; ++k) {
      int src = -1;
      size_t so = 0, dof = 0, len = 0;
      CHECK(plr_layout_segment(L, k, &src, &so, &dof, &len) == PLR_OK, "segment %d", k);
      CHECK(src >= 0 && src < W, "segment %d source %d", k, src);
      CHECK(so % 16 == 0 && dof % 16 == 0 && len % 16 == 0, "segment %d alignment", k);
      // (an empty segment moves nothing, wherever its offsets point)
      // (with explicit source offsets the caller sizes the sources)
      CHECK(len == 0 || d.in_offsets || so + len <= d.bytes_per_src, "segment %d reads [%zu, %zu) of %zu", k, so,
            so + len, d.bytes_per_src);
      CHECK(so + len >= so && dof + len >= dof, "segment %d offsets overflow", k);
      CHECK(len == 0 || dof + len <= dst_bytes, "segment %d writes [%zu, %zu) of %zu", k, dof, dof + len,
            dst_bytes);
      if (d.op == PLR_OP_COPY && len) outs.push_back({dof, dof + len});
    }
    std::sort(outs.begin(), outs.end());
    for (size_t k = 1; k < outs.size(); ++k)
      CHECK(outs[k - 1].second <= outs[k].first, "output segments overlap at %zu", outs[k].first);
    int src = 0;
    size_t so, dof, len;
    CHECK(plr_layout_segment(L, nseg, &src, &so, &dof, &len) == PLR_EINVAL, "segment past the end");
    CHECK(plr_layout_segment(L, -1, &src, &so, &dof, &len) == PLR_EINVAL, "negative segment");
    size_t tb = 0, cb = 0;
    int wg = -1, bl = 0, un = 0, st = 0, dp = 0, nm = 0;
    CHECK(plr_layout_policy(L, &tb, &cb, &wg, &bl, &un, &st, &dp, &nm) == PLR_OK, "policy");
    CHECK(plr_layout_policy(L, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == PLR_OK,
          "policy with NULL outputs");
    CHECK(tb % 16 == 0 && (tb > 0 || ntiles == 0), "tile %zu", tb);
    CHECK(cb % 16 == 0 && (ntiles == 0 || cb % tb == 0), "chunk %zu tile %zu", cb, tb);
    CHECK(bl == 64 || bl == 128 || bl == 256 || bl == 512, "block %d", bl);
    CHECK(un == 1 || un == 2 || un == 4, "unroll %d", un);
    CHECK(dp >= 1 && dp <= 3 && (nm == 1 || nm == 2) && wg >= 0, "datapath %d notify %d workgroups %d", dp, nm, wg);
    plr_layout_destroy(L);
  }
  const int it = iters;
  g_desc = nullptr;
  plr_layout_destroy(nullptr);
  CHECK(plr_layout_nsegments(nullptr) == -1 && plr_layout_dst_bytes(nullptr) == 0, "NULL layout queries");
  CHECK(accepted > iters / 20, "only %d of %d descriptors accepted", accepted, iters);
  printf("layout fuzz: %d descriptors, %d accepted\n", iters, accepted);
  return 0;
}
