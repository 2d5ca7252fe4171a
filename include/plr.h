/*
 * plr.h - C ABI of the single-GPU Atom datapath for gfx950 (AMD Instinct MI355X).
 *
 * The method is the datapath layer ("Atom") of Purlin (Aimuyo, Gandhi, Kozyrakis,
 * "Purlin: Separating Orchestration from the Datapath of Collectives"): two data
 * movement primitives, copy and reduce (abstract; section 3.3 "The Atom"), driven
 * by a collective specification that names an input layout, an output layout and
 * the copy or reduce operation (section 3.1 "Layouts"), and coordinated chunk by
 * chunk by Stage, Notify And Consume (section 3.2 "SNAC").
 *
 * This library runs one GPU's share of that work with the W contributions of the
 * W ranks held as W separate buffers in the same GPU's memory:
 *   - plr_reduce: elementwise sum of W contributions into one share
 *     (a ReduceScatter or AllReduce share), in source order 0..W-1;
 *   - plr_copy:   the layout copies of AllGather, AllToAll and the gather half
 *     of a composed AllReduce;
 *   - plr_copy_v: the variable-length AllToAll (MoE dispatch) packing.
 *
 * Conventions shared by every call
 *   - Pointers named "device" are HIP device pointers; "host" ones are host memory.
 *   - The caller owns every device buffer (sources, destination, counts, offsets,
 *     workspace, scratch). The library never allocates device memory; it owns only
 *     the host-side plr_layout object (and the fixed per-GPU scratch array in its
 *     device code that plr_copy_v_noalloc uses).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls that
 *     take a stream are asynchronous on it; plr_check is the only call that waits.
 *   - Alignment: every device address and every byte count must be a multiple of 16
 *     (the Atom's vector width; the reference implementation asks 16 bytes on all
 *     but its newest target, README "Using Purlin", Python note). Violations return
 *     PLR_EALIGN before anything is launched.
 *   - Errors are returned as int codes (PLR_OK = 0). Nothing aborts, and no C++
 *     exception crosses this ABI. Argument errors are detected on the host before
 *     any launch; on error the output buffers are untouched. PLR_EHIP reports a
 *     failed HIP launch (plr_last_hip_error gives the HIP code). A device-side
 *     notification timeout is sticky in the workspace and surfaces through plr_check.
 *   - Calls are not thread-safe on one plr_layout (its epoch advances per call);
 *     distinct layouts may be used from distinct threads.
 *   - Every call is kernel launches only (no memory-set or copy nodes), so calls can be
 *     captured in a HIP graph. A notified call (or a composed AllReduce) captured in a
 *     graph keeps the epoch it was captured with: replays do not wait for fresh
 *     notifications, so capture un-notified calls when replays must wait.
 */
#ifndef PLR_H
#define PLR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PLR_MAX_WORLD 16

/* ---- error codes ---- */
enum {
  PLR_OK = 0,
  PLR_EINVAL = 1,        /* bad argument: NULL, out of range, aliasing, bad layout pair */
  PLR_EALIGN = 2,        /* an address or byte count is not a multiple of 16 */
  PLR_EUNSUPPORTED = 3,  /* W > 16, a non-deterministic reduction mode, too many explicit segments */
  PLR_EHIP = 4,          /* a HIP runtime call or kernel launch failed */
  PLR_ETIMEOUT = 5,      /* device side: a chunk's notification did not arrive in time */
  PLR_ETOOLARGE = 6      /* the request exceeds the fixed scratch of an allocation-free entry point */
};

/* ---- element types (the reduction accumulates in binary32 for all of them) ---- */
typedef enum { PLR_BF16 = 0, PLR_F16 = 1, PLR_F32 = 2 } plr_dtype;

/* ---- the operation a collective applies between its layouts (section 3.1) ---- */
typedef enum { PLR_OP_REDUCE = 0, PLR_OP_COPY = 1, PLR_OP_ALLREDUCE = 2 } plr_op;

/* ---- layout kinds (section 3.1 "Layouts") ----
 * PACKED:     a rank's region is one contiguous block of bytes_per_src bytes.
 * SCATTERED:  a rank's region is W equal slices of bytes_per_src / W bytes;
 *             slice j belongs to rank j.
 * TRANSPOSED: a W x W grid of such slices in which output slice (d, s) is
 *             input slice (s, d).
 * Supported (in_kind, out_kind) pairs:
 *   reduce  PACKED    -> PACKED     the whole contribution is reduced (share = bytes_per_src)
 *   reduce  SCATTERED -> PACKED     rank `rank` reduces slice `rank` of every source
 *   copy    PACKED    -> PACKED     AllGather: source s lands at byte s * bytes_per_src
 *   copy    SCATTERED -> TRANSPOSED AllToAll: slice d of source s lands at slice d*W + s
 *   copy    SCATTERED -> SCATTERED  gather half of AllReduce: slice s of source s lands
 *                                   at slice s of the output
 *   allreduce SCATTERED -> SCATTERED  AllReduce = ReduceScatter then AllGather: every one
 *                                   of W outputs receives the reduction of all W sources
 * Variable-length variants (section 2.1, appendix C.4: contributions or partitions of
 * different sizes, given at run time), selected by part_bytes:
 *   reduce  SCATTERED -> PACKED     ReduceScatterV: every source holds W partitions of
 *                                   part_bytes[0..W-1] bytes back to back; rank `rank`
 *                                   reduces partition `rank` of every source
 *   copy    PACKED    -> PACKED     AllGatherV: source s contributes part_bytes[s] bytes,
 *                                   landing at the sum of the sizes before it
 */
typedef enum { PLR_PACKED = 0, PLR_SCATTERED = 1, PLR_TRANSPOSED = 2 } plr_layout_kind;

/* ---- datapath choice (section 3.3: the Atom's pipeline stages data through
 * workgroup-local memory; on gfx950 it can also go straight through registers) ---- */
enum { PLR_PATH_POLICY = 0, PLR_PATH_DIRECT = 1, PLR_PATH_LDS = 2, PLR_PATH_COMPOSED = 3 };

/* ---- how a notified call waits (section 3.2 "SNAC": a consumer never reads a chunk
 * before its flag). PLR_NOTIFY_CHUNKS: every workgroup waits for the flags of each
 * chunk it enters, then fences (agent-scope acquire). PLR_NOTIFY_CHECK: a one-workgroup
 * check kernel first reads all flags and records which have arrived; the consuming
 * kernel reads those chunks without waiting (the kernel boundary orders it after the
 * producers) and waits, as above, only for the chunks whose flags were still missing. ---- */
enum { PLR_NOTIFY_POLICY = 0, PLR_NOTIFY_CHUNKS = 1, PLR_NOTIFY_CHECK = 2 };

/* ---- reduction mode (README "Deterministic Reduction"): only the deterministic,
 * source-ordered reduction exists here. ---- */
enum { PLR_MODE_DETERMINISTIC = 0 };

/* A collective specification plus optional launch policy overrides.
 * Zero-initialise it, then fill the fields; every zero policy field means
 * "use the built-in gfx950 policy" (section 4.2 "Codesign Policies and Tuning":
 * chunk sizes, workgroup counts and pipeline depths are tuned per collective and
 * per GPU, and callers may supply their own). */
typedef struct {
  plr_op op;
  plr_dtype dtype;            /* element type; copies move bytes and ignore it */
  int world;                  /* W, number of sources, 1..16 */
  int rank;                   /* the share reduced by a SCATTERED reduce, 0..W-1 */
  size_t bytes_per_src;       /* bytes of each source buffer (multiple of 16, of 16*W if scattered) */
  plr_layout_kind in_kind, out_kind;
  /* Optional explicit byte offsets (multiples of 16) overriding the derived ones.
   * reduce: in_offsets[w] is where the share starts inside source w (W entries);
   *         out_offsets must be NULL.
   * copy:   one entry per segment in the derived segment order (source-major:
   *         W segments for AllGather / AllReduce gather, W*W for AllToAll with
   *         segment s*W + d); at most 64 segments; output segments must not overlap.
   * With explicit in_offsets a source must hold every byte its segments read (offset
   * plus length), which may reach past bytes_per_src; the library cannot see buffer
   * sizes. A segment whose end would pass 2^64 - 1 is PLR_EINVAL.
   * The arrays are copied at creation; the caller keeps ownership. */
  const size_t* in_offsets;
  const size_t* out_offsets;
  int mode;                   /* PLR_MODE_DETERMINISTIC (0); anything else: PLR_EUNSUPPORTED */
  /* policy overrides (0 = built-in policy) */
  size_t tile_bytes;          /* per-source bytes one workgroup consumes per step */
  size_t chunk_bytes;         /* per-source bytes one flag announces: the notification granule,
                                 rounded up to a whole number of tiles */
  int workgroups;             /* grid size; each workgroup then consumes a run of
                                 ceil(tiles / workgroups) consecutive tiles */
  int block;                  /* threads per workgroup: 64, 128, 256 or 512 */
  int unroll;                 /* 16-byte vectors per lane per pipeline step: 1, 2 or 4 (a reduce
                                 with W >= 15 takes at most 2: 4 x W vectors would not fit the
                                 registers; plr_layout_policy reports the value used) */
  int stages;                 /* reserved on input (1..4 accepted); plr_layout_policy reports the
                                 LDS ring depth: 4 stages for a reduce with W <= 4, 2 for more
                                 sources, 4 for a copy, 0 on the direct path */
  int datapath;               /* PLR_PATH_POLICY, PLR_PATH_DIRECT or PLR_PATH_LDS; the LDS path
                                 needs 256-thread workgroups and tiles of whole 4 KiB slabs */
  uint64_t spin_limit;        /* polls of a chunk flag before PLR_ETIMEOUT; 0 = default (about a second) */
  int notify_mode;            /* PLR_NOTIFY_POLICY (check first when some source contributes over
                                 2 MiB, in-kernel waits otherwise), PLR_NOTIFY_CHUNKS or
                                 PLR_NOTIFY_CHECK */
  int xcd_order;              /* 0 = policy (off), 1 = on, 2 = off: renumber workgroups so that each
                                 of the 8 XCDs walks one contiguous range of tiles */
  /* Variable-length layouts: W partition sizes in bytes (multiples of 16, zero allowed)
   * whose sum is the message size T, which bytes_per_src must equal; NULL = fixed
   * length. Copied at creation. A layout holds one set of sizes: for other sizes create
   * another (host work only). Only the two variable pairs above accept it, on the
   * direct datapath; a copy's offsets may still be overridden. */
  const size_t* part_bytes;
  /* Resident workgroups per compute unit for the layout's direct-path reduce, copy and fused
   * AllReduce launches, capped by reserving workgroup memory (LDS: 160 KiB per compute unit)
   * at each launch: 0 = policy (8 for the fused AllReduce of more than 2 MiB per source,
   * 1-4% faster than uncapped wherever its buffers sit; no cap elsewhere), -1 = no cap,
   * 1..16 = at most that many (one workgroup may hold all 160 KiB). The LDS-staged and
   * composed paths are never capped. 3 speeds that AllReduce by 8-14% over uncapped when its
   * sources and outputs fall on different places of the HBM address map (separately
   * allocated tensors of up to a few hundred MiB) and slows it by 10-25% when they collide
   * there (buffers a multiple of 512 MiB apart, some large allocations).
   * plr_layout_occupancy reports the cap used. */
  int wgs_per_cu;
} plr_layout_desc;

typedef struct plr_layout plr_layout; /* opaque, host only */

/* Compile a collective specification into a segment and chunk table
 * (sections 3.1 "Layouts" and 3.2 "SNAC": dependencies are derived from the
 * layouts). Host only: touches no device and allocates no device memory.
 * On success *out owns a new layout (free it with plr_layout_destroy) and the
 * layout's epoch is 0. Errors: PLR_EINVAL, PLR_EALIGN, PLR_EUNSUPPORTED. */
int plr_layout_create(const plr_layout_desc* desc, plr_layout** out);

/* Free a layout (NULL is accepted). */
void plr_layout_destroy(plr_layout* L);

/* Bytes of workspace a notified call needs: a 256-byte header (u64 error word at
 * byte 0, u64 ready word at byte 8, u64 late counter at byte 16), the chunk flags
 * uint64_t flags[F] and their
 * check-time mirror uint64_t mirror[F]. Reduce: F = W * nchunks, flags[w][c] for source
 * w and chunk c of the share. Copy: F = nchunks, one flag per chunk of every segment in
 * segment order (segment k's chunk j at k * nchunks / nsegments + j); segments go source
 * by source, so source s owns the s-th of W equal ranges. The caller allocates it in device
 * memory, ZEROED, once; it is never reset between calls (the epoch only grows,
 * section 4.3 "Epoch Bookkeeping"). One workspace belongs to one layout.
 * Diagnostics the caller may read: the ready word holds the epoch of the last call whose
 * check found every flag already set (0 if some were missing), mirror[i] that epoch if
 * flag i was set at check time (else 0), and the late counter grows by one for every
 * wait of a workgroup (or, for the composed AllReduce, a wave) that found a chunk flag
 * below its epoch and had to poll; the library never resets it. */
size_t plr_layout_workspace_bytes(const plr_layout* L);

/* Bytes the call writes into dst: the share for a reduce, the whole output for a copy
 * (0 for a NULL layout, as for plr_layout_workspace_bytes). */
size_t plr_layout_dst_bytes(const plr_layout* L);

/* Number of chunks (the notification granules), of tiles (workgroup steps) and of
 * copy segments; -1 for a NULL layout. */
int plr_layout_nchunks(const plr_layout* L);
int plr_layout_ntiles(const plr_layout* L);
int plr_layout_nsegments(const plr_layout* L);

/* Segment k of the compiled table, in bytes: the source index, the offset read in
 * that source, the offset written in dst, and the length. For a reduce there are W
 * segments (one per source, all with dst_off 0). Returns PLR_EINVAL if k is out of range. */
int plr_layout_segment(const plr_layout* L, int k, int* src, size_t* src_off,
                       size_t* dst_off, size_t* len);

/* The resolved launch policy (after the built-in table and the overrides).
 * workgroups == 0 means one workgroup per tile. Any output pointer may be NULL. */
int plr_layout_policy(const plr_layout* L, size_t* tile_bytes, size_t* chunk_bytes,
                      int* workgroups, int* block, int* unroll, int* stages, int* datapath,
                      int* notify_mode);

/* The launch shape of un-notified calls (plr_reduce / plr_copy with a NULL workspace):
 * bytes per tile, threads per workgroup and the tile count. They wait for no chunk, so a
 * reduce of at most 2 MiB per source on the direct datapath, with no tile, chunk or block
 * override, launches them with 4 KiB tiles of 256 threads whatever the notified shape;
 * every other layout reports its plr_layout_policy tile and block and plr_layout_ntiles.
 * The results are bitwise the same either way. Any output pointer may be NULL;
 * PLR_EINVAL for a NULL layout. */
int plr_layout_plain_shape(const plr_layout* L, size_t* tile_bytes, int* block, int* ntiles);

/* The resident-workgroup cap of the layout's direct-path launches (0 = none) and the
 * workgroup memory (LDS) each of those launches reserves for it, in bytes. Any output
 * pointer may be NULL; PLR_EINVAL for a NULL layout. */
int plr_layout_occupancy(const plr_layout* L, int* wgs_per_cu, size_t* lds_bytes);

/* Current epoch E of the layout: the last notified call consumed flags >= E (0 for a
 * NULL layout). */
uint64_t plr_layout_epoch(const plr_layout* L);

/* Reduce (section 3.3 "The Atom", SCORE): for every element i of the share,
 *   dst[i] = round(((x_0[i] + x_1[i]) + ...) + x_{W-1}[i])
 * with x_w the share inside srcs[w], binary32 accumulation starting from x_0, and
 * one round-to-nearest-even into the element type at the end. Each output element
 * is produced by one lane, sources in order, so the result is bitwise repeatable.
 *   srcs      host array of W device pointers (source w = rank w), each bytes_per_src bytes
 *             (with explicit in_offsets: up to the end of the bytes it reads)
 *   dst       device, plr_layout_dst_bytes(L) bytes; must not overlap any source share
 *   workspace device workspace of plr_layout_workspace_bytes(L), or NULL. When given,
 *             every chunk waits for flags[w][c] >= E+1 for all w (notify, section 3.2),
 *             and E advances by one after the launch.
 * Errors: PLR_EINVAL (NULL layout/pointer, wrong op, aliasing), PLR_EALIGN, PLR_EHIP. */
int plr_reduce(plr_layout* L, const void* const* srcs, void* dst, void* workspace, void* stream);

/* Copy (section 3.1 "Layouts", section 3.3 "The Atom"): moves every segment of the
 * layout's table, bytes only (NaN payloads and any bit pattern are preserved).
 *   srcs      host array of W device pointers, each bytes_per_src bytes (with explicit
 *             in_offsets: up to the end of the bytes its segments read)
 *   dst       device, plr_layout_dst_bytes(L) bytes; must not overlap any source
 *   workspace as for plr_reduce; a chunk of a segment waits only for its own
 *             source's flag.
 * Errors: as plr_reduce. */
int plr_copy(plr_layout* L, const void* const* srcs, void* dst, void* workspace, void* stream);

/* AllReduce of W contributions into W outputs (section 3.1 "Layouts": AllReduce is
 * ReduceScatter followed by AllGather, composed into one kernel; section 2.1: every
 * rank ends with the reduction of all contributions). The layout is op
 * PLR_OP_ALLREDUCE, SCATTERED -> SCATTERED, bytes_per_src a multiple of 16*W. For every
 * element i and every output w:
 *   dsts[w][i] = round(((x_0[i] + x_1[i]) + ...) + x_{W-1}[i])   (as plr_reduce)
 *   srcs      host array of W device pointers, bytes_per_src bytes each
 *   dsts      host array of W device pointers, bytes_per_src bytes each; they must not
 *             overlap each other or any source
 *   workspace datapath PLR_PATH_DIRECT (the policy's, "fused": each tile is reduced once
 *             and stored to all W outputs): NULL or any. PLR_PATH_COMPOSED (section 3.2's
 *             role split in one kernel: a workgroup reduces tile k into the output of
 *             the rank that owns k's slice and releases a per-tile flag, then acquires
 *             the flag of tile k-lag and copies that tile into the other W-1 outputs):
 *             required, plr_layout_workspace_bytes(L) bytes, zeroed once; the layout's
 *             epoch advances per call. Producer-side notification does not apply. All
 *             ntiles + 16 workgroups of a composed call must be resident at once (one per
 *             compute unit, 256): plr_layout_create refuses a composed layout whose tile_bytes
 *             override needs more with PLR_EUNSUPPORTED.
 * Errors: PLR_EINVAL (wrong op, NULL, overlaps, missing workspace), PLR_EALIGN, PLR_EHIP;
 * a composed call whose flags never arrive reports PLR_ETIMEOUT through plr_check. */
int plr_allreduce(plr_layout* L, const void* const* srcs, void* const* dsts, void* workspace,
                  void* stream);

/* Latency path (section 3.2 and Figure 7: for latency-bound transfers the producer
 * pushes packets that carry payload and notification together, doubling the data
 * volume, so the consumer needs no separate flag round trip; section 3.3: the packets
 * are reduced one output element per thread in source order). On gfx950 a packet is
 * one 8-byte atomic: a 4-byte payload word in the low half and the low 32 bits of the
 * epoch in the high half. Only for reduce layouts. plr_pack writes them from data already
 * in memory; a producing kernel can write them itself (include/plr_atom.h: packet_slot,
 * store_packet), which needs no separate pack or notify step.
 * plr_layout_packet_bytes: bytes of one source's packet buffer (4 x the share: two slots
 * of 2 x the share; epoch e packs into and is reduced from slot e & 1, section 4.3 "Epoch
 * Bookkeeping": the epoch's parity selects one of two staging buffers); the caller
 * allocates W of them in device memory, zeroed once, never reset.
 * Ordering: a producer may run one epoch ahead of the consumer (pack epoch e + 1 while
 * the consumer of epoch e still reads, the other slot), not two: packing epoch e + 2
 * reuses epoch e's slot, so it must wait until the consumer of epoch e has finished. */
size_t plr_layout_packet_bytes(const plr_layout* L);

/* Producer: stamp source src's share (src = -1: every source's, in one launch) with
 * epoch E+1 into its packet buffer, after the work queued on `stream`; E does not
 * change. data, packets: host arrays of W device pointers (source buffers, the layout's
 * offsets are applied; packet buffers); only the entries of the packed sources are read.
 * Errors: PLR_EINVAL (wrong op, src out of range, NULL, a packet buffer overlapping a
 * share or another packet buffer), PLR_EALIGN, PLR_EHIP. */
int plr_pack(plr_layout* L, int src, const void* const* data, void* const* packets, void* stream);

/* Consumer: for every output element, poll the W sources' packets until they carry
 * epoch E+1 (bounded; PLR_ETIMEOUT through plr_check), then reduce their payloads as
 * plr_reduce does; E advances by one. packets: host array of W device pointers.
 * workspace: device, at least 256 bytes, zeroed (the sticky error word).
 * Errors: PLR_EINVAL (wrong op, NULL, overlaps), PLR_EALIGN, PLR_EHIP. */
int plr_reduce_packets(plr_layout* L, const void* const* packets, void* dst, void* workspace,
                       void* stream);

/* Variable-length AllToAll packing (appendix C.4 "Variable-Length Collectives";
 * section 4: partition sizes at run time, prefix sums). Source s has rows_per_src[s]
 * rows of row_bytes bytes; row i goes to destination dest_of_row[s][i] in [0, W).
 *   counts[s*W + d]  (device, int64, W*W)  rows of source s bound for d
 *   offsets[d*W + s] (device, int64, W*W)  first output row of block (d, s):
 *                    destinations in order, and sources in order inside one
 *   dst (device, sum(rows) * row_bytes)    row i of source s lands at row
 *                    offsets[d*W + s] + (rows i' < i of source s bound for d)
 *   scratch (device, plr_copy_v_scratch_bytes bytes): zero it once before the first
 *            call; every call leaves its 256-byte header at zero again (the rest of
 *            it needs no initialisation). Concurrent calls need distinct scratch.
 *   srcs, dest_of_row: host arrays of W device pointers; rows_per_src: host array.
 * A destination id outside [0, W) is a caller error: its row is skipped and its
 * counts and offsets are undefined.
 * Errors: PLR_EINVAL (also an output of 2^64 bytes or more), PLR_EALIGN (row_bytes, srcs,
 * dst), PLR_EUNSUPPORTED (W > 16, or more than 2^31 - 1 rows in all), PLR_EHIP. */
int plr_copy_v(int world, const void* const* srcs, const int64_t* rows_per_src,
               const int32_t* const* dest_of_row, size_t row_bytes, void* dst,
               int64_t* counts, int64_t* offsets, void* scratch, void* stream);

/* Scratch bytes plr_copy_v needs for these row counts (host only): a 256-byte header,
 * one 32-bit key per row, and for every 1024-row segment of a source W int32 counts
 * and 16 int32 first output rows, each region rounded up to 256 bytes. 0 for invalid
 * arguments (W outside [1, 16], a negative row count) and for more than 2^31 - 1 rows
 * in all, which plr_copy_v does not support. */
size_t plr_copy_v_scratch_bytes(int world, const int64_t* rows_per_src);

/* Allocation-free form of plr_copy_v, for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid allocation):
 * the same operation, arguments and results as plr_copy_v, without the scratch
 * argument. Its scratch is a fixed array of plr_copy_v_noalloc_max_scratch_bytes()
 * bytes (4 MiB) in the library's device code, one per GPU, held until the process ends;
 * no call allocates or frees memory. A request whose plr_copy_v_scratch_bytes exceeds
 * that size (about a million rows in all) returns PLR_ETOOLARGE and launches nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different threads) race and must not be issued. The
 * kernels run on the stream's device (the current device for the NULL stream).
 * Errors: as plr_copy_v, plus PLR_ETOOLARGE. */
int plr_copy_v_noalloc(int world, const void* const* srcs, const int64_t* rows_per_src,
                       const int32_t* const* dest_of_row, size_t row_bytes, void* dst,
                       int64_t* counts, int64_t* offsets, void* stream);

/* Size in bytes of plr_copy_v_noalloc's fixed scratch. */
size_t plr_copy_v_noalloc_max_scratch_bytes(void);

/* Producer side of notify (section 3.2 "SNAC"; section 4.3: the epoch supplies the
 * notification value): release-stores E+1 into every chunk flag of source `src`
 * (or of all sources if src == -1), after all work already queued on `stream`.
 * The next plr_reduce / plr_copy on L consumes epoch E+1.
 * Ordering: the sources are single-buffered. A consumer accepts any flag >= its epoch,
 * so a producer must not write a source's next contents (or notify epoch E+2) before the
 * call consuming E+1 has finished reading it; order that rewrite after the call (stream
 * order, or an event recorded after it). Packets keep two slots per source so that a
 * producer may run one epoch ahead (plr_pack).
 * Errors: PLR_EINVAL (src out of range, NULL workspace), PLR_EALIGN, PLR_EHIP. */
int plr_notify(plr_layout* L, int src, void* workspace, void* stream);

/* Wait for `stream`, then read and clear the workspace's sticky device error.
 * Returns PLR_OK, PLR_ETIMEOUT (some chunk's flag never reached its epoch; that
 * call's output is undefined), or PLR_EHIP / PLR_EINVAL for the check itself. */
int plr_check(plr_layout* L, void* workspace, void* stream);

/* Measurement aid (not part of the method): while `before` and `after` are set, every
 * datapath call made by the calling host thread (plr_reduce, plr_copy, plr_copy_v,
 * plr_allreduce, plr_reduce_packets) launches its first datapath kernel with `before`
 * and its last with `after` as that dispatch's start and end events
 * (hipExtLaunchKernel), so the pair times the datapath kernels alone, as a kernel
 * trace does: a notified call's check kernel is outside it. A call that launches no
 * datapath kernel (an empty layout) records neither. Both are hipEvent_t handles the
 * caller owns and has created; NULL, NULL turns this off. The setting is per host
 * thread and is not for calls captured into a graph. Errors: PLR_EINVAL if exactly one
 * of the two is NULL. */
int plr_set_timing_events(void* before, void* after);

/* Measurement aid, as plr_set_timing_events, for calls of two datapath kernels (the
 * variable-length AllToAll's rank and scatter kernels): the first dispatch carries
 * `before` and `first_after` as its start and end events, the last carries
 * `last_before` and `after`, so the two durations can be summed without the time
 * between the dispatches (timing the first dispatch delays the next one). A call of one
 * datapath kernel records only `before` and `after` on it. Errors: PLR_EINVAL unless
 * all four are NULL (off) or none is. */
int plr_set_timing_events_split(void* before, void* first_after, void* last_before, void* after);

/* Static text for an error code. */
const char* plr_strerror(int code);

/* The HIP error code of the last PLR_EHIP on this thread (0 if none). */
int plr_last_hip_error(void);

/* Library version string. */
const char* plr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PLR_H */
