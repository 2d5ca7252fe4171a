"""Python binding of libplr.so: the single-GPU Atom datapath (copy and reduce) for gfx950.

Argument marshalling only: every step of the datapath runs in the library's HIP
kernels. The functions carry the C ABI's names (include/plr.h) and take torch
tensors (device memory) or raw integer device addresses. torch supplies memory and
streams; nothing here computes.

Importing this package loads ``libplr.so`` from this directory and raises
ImportError if it has not been built (``python reduce_atom_amd/_build.py``): there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libplr.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python reduce_atom_amd/_build.py`")

# libplr.so must run on the HIP runtime that owns torch's memory and streams. torch
# loads its bundled libamdhip64 by file name, so if libplr.so came first, its own
# dependency (the system ROCm runtime, same soname) would be loaded and torch would
# then load a second runtime beside it: the library's launches would go to a runtime
# that owns neither torch's memory nor its streams.
# Importing torch first makes libplr.so bind to torch's runtime.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

# ---- constants (include/plr.h) ----
PLR_OK, PLR_EINVAL, PLR_EALIGN, PLR_EUNSUPPORTED, PLR_EHIP, PLR_ETIMEOUT, PLR_ETOOLARGE = range(7)
PLR_BF16, PLR_F16, PLR_F32 = 0, 1, 2
PLR_OP_REDUCE, PLR_OP_COPY, PLR_OP_ALLREDUCE = 0, 1, 2
PLR_PACKED, PLR_SCATTERED, PLR_TRANSPOSED = 0, 1, 2
PLR_PATH_POLICY, PLR_PATH_DIRECT, PLR_PATH_LDS, PLR_PATH_COMPOSED = 0, 1, 2, 3
PLR_MODE_DETERMINISTIC = 0
PLR_NOTIFY_POLICY, PLR_NOTIFY_CHUNKS, PLR_NOTIFY_CHECK = 0, 1, 2
PLR_MAX_WORLD = 16

DTYPE_CODES = {"bf16": PLR_BF16, "f16": PLR_F16, "f32": PLR_F32}
KIND_CODES = {"packed": PLR_PACKED, "scattered": PLR_SCATTERED, "transposed": PLR_TRANSPOSED}
OP_CODES = {"reduce": PLR_OP_REDUCE, "copy": PLR_OP_COPY, "allreduce": PLR_OP_ALLREDUCE}

_c = ctypes
_vp, _sz, _i, _u64, _i64p = _c.c_void_p, _c.c_size_t, _c.c_int, _c.c_uint64, _c.POINTER(_c.c_int64)


class plr_layout_desc(_c.Structure):
    _fields_ = [
        ("op", _i), ("dtype", _i), ("world", _i), ("rank", _i),
        ("bytes_per_src", _sz),
        ("in_kind", _i), ("out_kind", _i),
        ("in_offsets", _c.POINTER(_sz)), ("out_offsets", _c.POINTER(_sz)),
        ("mode", _i),
        ("tile_bytes", _sz), ("chunk_bytes", _sz),
        ("workgroups", _i), ("block", _i), ("unroll", _i), ("stages", _i), ("datapath", _i),
        ("spin_limit", _u64),
        ("notify_mode", _i),
        ("xcd_order", _i),
        ("part_bytes", _c.POINTER(_sz)),
        ("wgs_per_cu", _i),
    ]


_lib.plr_layout_create.argtypes = [_c.POINTER(plr_layout_desc), _c.POINTER(_vp)]
_lib.plr_layout_create.restype = _i
_lib.plr_layout_destroy.argtypes = [_vp]
_lib.plr_layout_destroy.restype = None
for _n in ("plr_layout_workspace_bytes", "plr_layout_dst_bytes"):
    getattr(_lib, _n).argtypes = [_vp]
    getattr(_lib, _n).restype = _sz
for _n in ("plr_layout_nchunks", "plr_layout_ntiles", "plr_layout_nsegments"):
    getattr(_lib, _n).argtypes = [_vp]
    getattr(_lib, _n).restype = _i
_lib.plr_layout_epoch.argtypes = [_vp]
_lib.plr_layout_epoch.restype = _u64
_lib.plr_layout_segment.argtypes = [_vp, _i, _c.POINTER(_i), _c.POINTER(_sz), _c.POINTER(_sz),
                                    _c.POINTER(_sz)]
_lib.plr_layout_segment.restype = _i
_lib.plr_layout_policy.argtypes = [_vp, _c.POINTER(_sz), _c.POINTER(_sz)] + [_c.POINTER(_i)] * 6
_lib.plr_layout_policy.restype = _i
_lib.plr_layout_plain_shape.argtypes = [_vp, _c.POINTER(_sz), _c.POINTER(_i), _c.POINTER(_i)]
_lib.plr_layout_plain_shape.restype = _i
_lib.plr_layout_occupancy.argtypes = [_vp, _c.POINTER(_i), _c.POINTER(_sz)]
_lib.plr_layout_occupancy.restype = _i
_lib.plr_reduce.argtypes = [_vp, _c.POINTER(_vp), _vp, _vp, _vp]
_lib.plr_reduce.restype = _i
_lib.plr_copy.argtypes = [_vp, _c.POINTER(_vp), _vp, _vp, _vp]
_lib.plr_copy.restype = _i
_lib.plr_allreduce.argtypes = [_vp, _c.POINTER(_vp), _c.POINTER(_vp), _vp, _vp]
_lib.plr_allreduce.restype = _i
_lib.plr_layout_packet_bytes.argtypes = [_vp]
_lib.plr_layout_packet_bytes.restype = _sz
_lib.plr_pack.argtypes = [_vp, _i, _c.POINTER(_vp), _c.POINTER(_vp), _vp]
_lib.plr_pack.restype = _i
_lib.plr_reduce_packets.argtypes = [_vp, _c.POINTER(_vp), _vp, _vp, _vp]
_lib.plr_reduce_packets.restype = _i
_lib.plr_copy_v.argtypes = [_i, _c.POINTER(_vp), _i64p, _c.POINTER(_vp), _sz, _vp, _vp, _vp, _vp, _vp]
_lib.plr_copy_v.restype = _i
_lib.plr_copy_v_scratch_bytes.argtypes = [_i, _i64p]
_lib.plr_copy_v_scratch_bytes.restype = _sz
_lib.plr_copy_v_noalloc.argtypes = [_i, _c.POINTER(_vp), _i64p, _c.POINTER(_vp), _sz, _vp, _vp, _vp, _vp]
_lib.plr_copy_v_noalloc.restype = _i
_lib.plr_copy_v_noalloc_max_scratch_bytes.argtypes = []
_lib.plr_copy_v_noalloc_max_scratch_bytes.restype = _sz
_lib.plr_notify.argtypes = [_vp, _i, _vp, _vp]
_lib.plr_notify.restype = _i
_lib.plr_check.argtypes = [_vp, _vp, _vp]
_lib.plr_check.restype = _i
_lib.plr_set_timing_events.argtypes = [_vp, _vp]
_lib.plr_set_timing_events.restype = _i
_lib.plr_set_timing_events_split.argtypes = [_vp, _vp, _vp, _vp]
_lib.plr_set_timing_events_split.restype = _i
_lib.plr_strerror.argtypes = [_i]
_lib.plr_strerror.restype = _c.c_char_p
_lib.plr_last_hip_error.argtypes = []
_lib.plr_last_hip_error.restype = _i
_lib.plr_version.argtypes = []
_lib.plr_version.restype = _c.c_char_p

EXPORTS = [
    "plr_layout_create", "plr_layout_destroy", "plr_layout_workspace_bytes", "plr_layout_dst_bytes",
    "plr_layout_nchunks", "plr_layout_ntiles", "plr_layout_nsegments", "plr_layout_segment", "plr_layout_policy",
    "plr_layout_plain_shape", "plr_layout_occupancy",
    "plr_layout_epoch", "plr_reduce", "plr_copy", "plr_allreduce", "plr_copy_v", "plr_copy_v_scratch_bytes",
    "plr_copy_v_noalloc", "plr_copy_v_noalloc_max_scratch_bytes",
    "plr_layout_packet_bytes", "plr_pack", "plr_reduce_packets",
    "plr_notify", "plr_check", "plr_set_timing_events", "plr_set_timing_events_split", "plr_strerror",
    "plr_last_hip_error",
    "plr_version",
]


class PlrError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = plr_strerror(code)
        if code == PLR_EHIP:
            msg += f" (hip error {_lib.plr_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{code}]")


def _ok(rc: int, where: str) -> None:
    if rc != PLR_OK:
        raise PlrError(rc, where)


def plr_strerror(code: int) -> str:
    return _lib.plr_strerror(code).decode()


def plr_version() -> str:
    return _lib.plr_version().decode()


def _addr(x) -> int | None:
    """Device address of a tensor (contiguous, on a GPU) or a raw integer address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("device tensor expected")
    if not x.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptrs(xs):
    return (_vp * len(xs))(*[_addr(x) for x in xs])


def _check_len(xs, n: int, what: str) -> None:
    if xs is not None and len(xs) != n:
        raise ValueError(f"{what}: {len(xs)} entries, the layout reads {n}")


def _world_ptrs(layout: "Layout", xs, what: str):
    """One device pointer per source of the layout (the C side reads exactly W)."""
    _check_len(xs, layout.world, what)
    return _ptrs(xs)


def _need(x, nbytes: int, what: str) -> None:
    """A tensor argument holds at least the `nbytes` bytes the call reads or writes
    through it (the C side takes bare pointers and cannot check); raw integer
    addresses and None are the caller's responsibility."""
    if x is None or isinstance(x, int):
        return
    have = x.numel() * x.element_size()
    if have < nbytes:
        raise ValueError(f"{what}: {have} bytes, the call uses {nbytes}")


def _need_each(xs, sizes, what: str) -> None:
    for w, (x, n) in enumerate(zip(xs, sizes)):
        _need(x, n, f"{what}[{w}]")


class Layout:
    """A compiled collective specification (host object owning a plr_layout*)."""

    def __init__(self, handle: int, world: int = 0):
        self._h = _vp(handle)
        self.world = world

    @property
    def handle(self):
        return self._h

    def __del__(self, _destroy=_lib.plr_layout_destroy):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _destroy(h)
            self._h = None

    @property
    def workspace_bytes(self) -> int:
        return _lib.plr_layout_workspace_bytes(self._h)

    @property
    def dst_bytes(self) -> int:
        return _lib.plr_layout_dst_bytes(self._h)

    @property
    def nchunks(self) -> int:
        return _lib.plr_layout_nchunks(self._h)

    @property
    def epoch(self) -> int:
        return _lib.plr_layout_epoch(self._h)

    def segments(self):
        out = []
        for k in range(_lib.plr_layout_nsegments(self._h)):
            s, so, do, ln = _i(), _sz(), _sz(), _sz()
            _ok(_lib.plr_layout_segment(self._h, k, _c.byref(s), _c.byref(so), _c.byref(do),
                                        _c.byref(ln)), "plr_layout_segment")
            out.append((s.value, so.value, do.value, ln.value))
        return out

    @property
    def packet_bytes(self) -> int:
        return _lib.plr_layout_packet_bytes(self._h)

    def src_extent(self) -> list:
        """Bytes of each source the layout's segments reach (its furthest segment end)."""
        if getattr(self, "_extent", None) is None:
            ext = [0] * self.world
            for s, so, _do, ln in self.segments():
                if ln:
                    ext[s] = max(ext[s], so + ln)
            self._extent = ext
        return self._extent

    @property
    def ntiles(self) -> int:
        return _lib.plr_layout_ntiles(self._h)

    def policy(self) -> dict:
        tb, cb, wg, bl, un, st, dp, nm = _sz(), _sz(), _i(), _i(), _i(), _i(), _i(), _i()
        _ok(_lib.plr_layout_policy(self._h, _c.byref(tb), _c.byref(cb), _c.byref(wg), _c.byref(bl),
                                   _c.byref(un), _c.byref(st), _c.byref(dp), _c.byref(nm)),
            "plr_layout_policy")
        pt, pb, pn = _sz(), _i(), _i()
        _ok(_lib.plr_layout_plain_shape(self._h, _c.byref(pt), _c.byref(pb), _c.byref(pn)),
            "plr_layout_plain_shape")
        oc, ol = _i(), _sz()
        _ok(_lib.plr_layout_occupancy(self._h, _c.byref(oc), _c.byref(ol)), "plr_layout_occupancy")
        return dict(tile_bytes=tb.value, chunk_bytes=cb.value, workgroups=wg.value, block=bl.value,
                    unroll=un.value, stages=st.value, datapath=dp.value, notify_mode=nm.value,
                    plain_tile_bytes=pt.value, plain_block=pb.value, plain_ntiles=pn.value,
                    wgs_per_cu=oc.value, lds_reserve=ol.value)


def plr_layout_create(op, dtype, world, bytes_per_src, in_kind, out_kind, rank=0,
                      in_offsets=None, out_offsets=None, mode=PLR_MODE_DETERMINISTIC,
                      tile_bytes=0, chunk_bytes=0, workgroups=0, block=0, unroll=0, stages=0, datapath=0,
                      spin_limit=0, notify_mode=0, xcd_order=0, part_bytes=None, wgs_per_cu=0) -> Layout:
    """Compile a layout. op/dtype/kinds accept the C enum values or their names.
    part_bytes: W partition sizes of a variable-length layout (AllGatherV, ReduceScatterV).
    wgs_per_cu: resident workgroups per compute unit (0 policy, -1 no cap, 1..16)."""
    d = plr_layout_desc()
    op_c, in_c, out_c = OP_CODES.get(op, op), KIND_CODES.get(in_kind, in_kind), KIND_CODES.get(out_kind, out_kind)
    # the C side reads exactly this many entries of every list it is given
    if isinstance(world, int) and 1 <= world <= PLR_MAX_WORLD:
        # (a reduce rejects out_offsets and an AllReduce both lists without reading them)
        nseg = world * world if (op_c, in_c, out_c) == (PLR_OP_COPY, PLR_SCATTERED, PLR_TRANSPOSED) else world
        if op_c in (PLR_OP_REDUCE, PLR_OP_COPY):
            _check_len(in_offsets, nseg, "in_offsets")
        if op_c == PLR_OP_COPY:
            _check_len(out_offsets, nseg, "out_offsets")
        _check_len(part_bytes, world, "part_bytes")
    d.op = op_c
    d.dtype = DTYPE_CODES.get(dtype, dtype)
    d.world, d.rank, d.bytes_per_src = world, rank, bytes_per_src
    d.in_kind = KIND_CODES.get(in_kind, in_kind)
    d.out_kind = KIND_CODES.get(out_kind, out_kind)
    keep = []
    if in_offsets is not None:
        a = (_sz * len(in_offsets))(*in_offsets)
        keep.append(a)
        d.in_offsets = _c.cast(a, _c.POINTER(_sz))
    if out_offsets is not None:
        a = (_sz * len(out_offsets))(*out_offsets)
        keep.append(a)
        d.out_offsets = _c.cast(a, _c.POINTER(_sz))
    d.mode, d.tile_bytes, d.chunk_bytes, d.workgroups = mode, tile_bytes, chunk_bytes, workgroups
    d.block, d.unroll, d.stages, d.datapath, d.spin_limit = block, unroll, stages, datapath, spin_limit
    d.notify_mode = notify_mode
    d.xcd_order = xcd_order
    d.wgs_per_cu = wgs_per_cu
    if part_bytes is not None:
        a = (_sz * len(part_bytes))(*part_bytes)
        keep.append(a)
        d.part_bytes = _c.cast(a, _c.POINTER(_sz))
    h = _vp()
    _ok(_lib.plr_layout_create(_c.byref(d), _c.byref(h)), "plr_layout_create")
    return Layout(h.value, world)


def plr_layout_destroy(layout: Layout) -> None:
    layout.__del__()


def _check_sizes(layout: Layout, srcs, dst, workspace) -> None:
    if srcs is not None and len(srcs) == layout.world:
        _need_each(srcs, layout.src_extent(), "srcs")
    _need(dst, layout.dst_bytes, "dst")
    if workspace is not None:
        _need(workspace, layout.workspace_bytes, "workspace")


def plr_reduce(layout: Layout, srcs, dst, workspace=None, stream=None) -> None:
    _check_sizes(layout, srcs, dst, workspace)
    _ok(_lib.plr_reduce(layout.handle, _world_ptrs(layout, srcs, "srcs"), _addr(dst), _addr(workspace),
                        _stream(stream)), "plr_reduce")


def plr_copy(layout: Layout, srcs, dst, workspace=None, stream=None) -> None:
    _check_sizes(layout, srcs, dst, workspace)
    _ok(_lib.plr_copy(layout.handle, _world_ptrs(layout, srcs, "srcs"), _addr(dst), _addr(workspace),
                      _stream(stream)), "plr_copy")


def plr_allreduce(layout: Layout, srcs, dsts, workspace=None, stream=None) -> None:
    # the fused datapath ignores the workspace; the composed one keeps its flags there
    composed = layout.policy()["datapath"] == PLR_PATH_COMPOSED
    _check_sizes(layout, srcs, None, workspace if composed else None)
    if dsts is not None and len(dsts) == layout.world:
        _need_each(dsts, [layout.dst_bytes] * layout.world, "dsts")
    _ok(_lib.plr_allreduce(layout.handle, _world_ptrs(layout, srcs, "srcs"), _world_ptrs(layout, dsts, "dsts"),
                           _addr(workspace), _stream(stream)), "plr_allreduce")


def plr_pack(layout: Layout, src: int, data, packets, stream=None) -> None:
    if data is not None and packets is not None and len(data) == len(packets) == layout.world:
        ext = layout.src_extent()
        for w in range(layout.world) if src == -1 else ([src] if 0 <= src < layout.world else []):
            _need(data[w], ext[w], f"data[{w}]")
            _need(packets[w], layout.packet_bytes, f"packets[{w}]")
    _ok(_lib.plr_pack(layout.handle, src, _world_ptrs(layout, data, "data"), _world_ptrs(layout, packets, "packets"),
                      _stream(stream)), "plr_pack")


def plr_reduce_packets(layout: Layout, packets, dst, workspace, stream=None) -> None:
    if packets is not None and len(packets) == layout.world:
        _need_each(packets, [layout.packet_bytes] * layout.world, "packets")
    _need(dst, layout.dst_bytes, "dst")
    _need(workspace, 256, "workspace")
    _ok(_lib.plr_reduce_packets(layout.handle, _world_ptrs(layout, packets, "packets"), _addr(dst),
                                _addr(workspace), _stream(stream)), "plr_reduce_packets")


def plr_copy_v_scratch_bytes(world: int, rows_per_src) -> int:
    _check_len(rows_per_src, world, "rows_per_src")
    rows = (_c.c_int64 * world)(*rows_per_src)
    return _lib.plr_copy_v_scratch_bytes(world, rows)


def _copy_v_lists(srcs, rows_per_src, dest_of_row):
    W = len(srcs)
    _check_len(rows_per_src, W, "rows_per_src")
    _check_len(dest_of_row, W, "dest_of_row")
    for d in dest_of_row:
        dt = getattr(d, "dtype", None)
        if dt is not None and str(dt) != "torch.int32":
            raise ValueError(f"dest_of_row: int32 tensors expected, got {dt}")
    return W, (_c.c_int64 * W)(*rows_per_src)


def _copy_v_sizes(W, rows_per_src, srcs, dest_of_row, row_bytes, dst, counts, offsets) -> None:
    if any(r < 0 for r in rows_per_src) or row_bytes < 0:
        return  # the library rejects these itself
    _need_each(srcs, [r * row_bytes for r in rows_per_src], "srcs")
    _need_each(dest_of_row, [4 * r for r in rows_per_src], "dest_of_row")
    _need(dst, sum(rows_per_src) * row_bytes, "dst")
    _need(counts, 8 * W * W, "counts")
    _need(offsets, 8 * W * W, "offsets")


def plr_copy_v(srcs, rows_per_src, dest_of_row, row_bytes, dst, counts, offsets, scratch,
               stream=None) -> None:
    W, rows = _copy_v_lists(srcs, rows_per_src, dest_of_row)
    _copy_v_sizes(W, rows_per_src, srcs, dest_of_row, row_bytes, dst, counts, offsets)
    if 1 <= W <= PLR_MAX_WORLD:
        _need(scratch, plr_copy_v_scratch_bytes(W, rows_per_src), "scratch")
    _ok(_lib.plr_copy_v(W, _ptrs(srcs), rows, _ptrs(dest_of_row), row_bytes, _addr(dst),
                        _addr(counts), _addr(offsets), _addr(scratch), _stream(stream)), "plr_copy_v")


def plr_copy_v_noalloc(srcs, rows_per_src, dest_of_row, row_bytes, dst, counts, offsets, stream=None) -> None:
    """plr_copy_v with the library's fixed per-GPU scratch instead of a caller buffer."""
    W, rows = _copy_v_lists(srcs, rows_per_src, dest_of_row)
    _copy_v_sizes(W, rows_per_src, srcs, dest_of_row, row_bytes, dst, counts, offsets)
    _ok(_lib.plr_copy_v_noalloc(W, _ptrs(srcs), rows, _ptrs(dest_of_row), row_bytes, _addr(dst),
                                _addr(counts), _addr(offsets), _stream(stream)), "plr_copy_v_noalloc")


def plr_copy_v_noalloc_max_scratch_bytes() -> int:
    return _lib.plr_copy_v_noalloc_max_scratch_bytes()


def plr_notify(layout: Layout, src: int, workspace, stream=None) -> None:
    _need(workspace, layout.workspace_bytes, "workspace")
    _ok(_lib.plr_notify(layout.handle, src, _addr(workspace), _stream(stream)), "plr_notify")


def plr_set_timing_events(before=None, after=None) -> None:
    """Bracket the datapath kernels of this thread's next calls with two events: raw
    hipEvent_t handles (int) or torch.cuda.Event objects made with enable_timing=True
    (recorded once here if torch has not created their HIP event yet). No arguments
    turns it off."""
    if before is None and after is None:
        _ok(_lib.plr_set_timing_events(None, None), "plr_set_timing_events")
        return

    def handle(e):
        if isinstance(e, int):
            return e
        if not e.cuda_event:  # torch creates its HIP event at the first record
            e.record()
        return e.cuda_event

    _ok(_lib.plr_set_timing_events(handle(before), handle(after)), "plr_set_timing_events")


def plr_set_timing_events_split(before=None, first_after=None, last_before=None, after=None) -> None:
    """Four raw hipEvent_t handles (int): the first datapath dispatch of this thread's
    next calls carries before / first_after, the last carries last_before / after. No
    arguments turns it off."""
    _ok(_lib.plr_set_timing_events_split(before, first_after, last_before, after), "plr_set_timing_events_split")


def plr_check(layout: Layout, workspace, stream=None) -> int:
    """Returns the sticky device error code (PLR_OK or PLR_ETIMEOUT) and clears it."""
    return _lib.plr_check(layout.handle, _addr(workspace), _stream(stream))
