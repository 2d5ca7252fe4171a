"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports every
symbol include/plr.h declares, its struct layout matches the binding, and the layout
compiler, policy and argument validation behave as the header states. No call here
reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT, golden_lines


@pytest.fixture(scope="module")
def plr():
    so = os.path.join(ROOT, "reduce_atom_amd", "libplr.so")
    if not os.path.exists(so):
        import __graft_entry__

        __graft_entry__._load_builder().build()
    import reduce_atom_amd

    return reduce_atom_amd


def _declared_functions():
    with open(os.path.join(ROOT, "include", "plr.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(plr_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(plr):
    names = _declared_functions()
    assert len(names) >= 18
    lib = ctypes.CDLL(plr.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(plr.EXPORTS) == names
    out = subprocess.run(["nm", "-D", "--defined-only", plr.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (plr_\w+)", out))
    assert exported == set(names)


def test_desc_struct_layout_matches_c(plr, tmp_path):
    fields = [f for f, _ in plr.plr_layout_desc._fields_]
    prog = tmp_path / "abi.c"
    prog.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"plr.h\"\nint main(void){\n"
                    "printf(\"%zu\\n\", sizeof(plr_layout_desc));\n"
                    + "".join(f"printf(\"%zu\\n\", offsetof(plr_layout_desc, {f}));\n" for f in fields)
                    + "return 0;}\n")
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(plr.plr_layout_desc)
    assert got[1:] == [getattr(plr.plr_layout_desc, f).offset for f in fields]


def test_segments_match_golden(plr):
    for line in golden_lines("layout_segments.txt"):
        ik, ok, *segs = line.split()
        want = sorted(tuple(int(v) for v in s.split(":")) for s in segs)
        L = plr.plr_layout_create("copy", "bf16", 2, 32, ik, ok)
        assert sorted(L.segments()) == want, line


@pytest.mark.parametrize("W", [1, 2, 3, 8, 9, 16])
@pytest.mark.parametrize("pair", [("packed", "packed"), ("scattered", "transposed"),
                                  ("scattered", "scattered")])
def test_segments_match_oracle_reading(plr, oracle_mod, W, pair):
    B = 16 * W * 5
    L = plr.plr_layout_create("copy", "bf16", W, B, *pair)
    ref, total = oracle_mod.copy_segments(pair[0], pair[1], W, B)
    assert sorted(L.segments()) == sorted(ref)
    assert L.dst_bytes == total


@pytest.mark.parametrize("W,rank", [(1, 0), (4, 0), (4, 3), (8, 5)])
def test_reduce_share_segments(plr, oracle_mod, W, rank):
    B = 16 * W * 7
    L = plr.plr_layout_create("reduce", "bf16", W, B, "scattered", "packed", rank=rank)
    offs, n = oracle_mod.reduce_share("scattered", W, rank, B // 2)
    assert L.segments() == [(w, offs[w] * 2, 0, n * 2) for w in range(W)]
    assert L.dst_bytes == n * 2
    P = plr.plr_layout_create("reduce", "f32", W, B, "packed", "packed")
    assert P.segments() == [(w, 0, 0, B) for w in range(W)]


def test_chunks_and_workspace(plr):
    L = plr.plr_layout_create("reduce", "bf16", 8, 8192 * 7168 * 2, "packed", "packed")
    pol = L.policy()
    n = -(-8192 * 7168 * 2 // pol["chunk_bytes"])
    assert L.nchunks == n
    assert L.workspace_bytes == 256 + 2 * 8 * n * 8
    C = plr.plr_layout_create("copy", "bf16", 8, 64 << 20, "scattered", "transposed", chunk_bytes=1 << 20)
    # copy flags: one per chunk of every segment (not per source and chunk)
    assert C.nchunks == 64 * 8 and C.workspace_bytes == 256 + 2 * 512 * 8
    R = plr.plr_layout_create("copy", "bf16", 3, 48 * 3, "packed", "packed", chunk_bytes=32)
    assert R.nchunks == 3 * 5  # 144-byte segments in 32-byte chunks: ragged last chunk
    E = plr.plr_layout_create("reduce", "bf16", 4, 0, "packed", "packed")
    assert E.nchunks == 0 and E.dst_bytes == 0


def test_policy_overrides(plr):
    L = plr.plr_layout_create("reduce", "f16", 4, 1 << 24, "packed", "packed", chunk_bytes=4096,
                              workgroups=33, block=128, unroll=4, datapath=plr.PLR_PATH_DIRECT)
    assert L.policy() == dict(tile_bytes=2048, chunk_bytes=4096, workgroups=33, block=128, unroll=4,
                              stages=0, datapath=plr.PLR_PATH_DIRECT, notify_mode=plr.PLR_NOTIFY_CHECK,
                              plain_tile_bytes=2048, plain_block=128, plain_ntiles=8192,
                              wgs_per_cu=0, lds_reserve=0)
    # the LDS path reports its ring depth: W KiB per stage per wave for a reduce
    for w, depth in ((1, 4), (4, 4), (5, 2), (8, 2), (9, 2), (16, 2)):
        R = plr.plr_layout_create("reduce", "bf16", w, 1 << 20, "packed", "packed", datapath=plr.PLR_PATH_LDS)
        assert R.policy()["stages"] == depth and R.policy()["block"] == 256
    C = plr.plr_layout_create("copy", "bf16", 8, 1 << 20, "packed", "packed", datapath=plr.PLR_PATH_LDS)
    assert C.policy()["stages"] == 4 and C.policy()["tile_bytes"] == 4096
    S = plr.plr_layout_create("reduce", "bf16", 8, 7168 * 2, "packed", "packed")
    assert S.policy()["notify_mode"] == plr.PLR_NOTIFY_CHUNKS  # decode-size share
    M = plr.plr_layout_create("reduce", "bf16", 8, 7168 * 2, "packed", "packed", notify_mode=plr.PLR_NOTIFY_CHECK)
    assert M.policy()["notify_mode"] == plr.PLR_NOTIFY_CHECK
    assert _code(plr.plr_layout_create, "reduce", "bf16", 8, 64, "packed", "packed", notify_mode=3) == plr.PLR_EINVAL


def test_regime_follows_bytes_per_source(plr):
    # over 2 MiB from some source: check first, and copies take 4 KiB tiles; else in-kernel
    # waits and 2 KiB tiles. An AllToAll's segments are slices, its sources contribute W of them.
    def pol(*a, **k):
        return plr.plr_layout_create(*a, **k).policy()
    a2a = pol("copy", "bf16", 8, 4 << 20, "scattered", "transposed")  # 512 KiB slices
    assert a2a["notify_mode"] == plr.PLR_NOTIFY_CHECK and a2a["tile_bytes"] == 4096
    ag = pol("copy", "bf16", 8, 2 << 20, "packed", "packed")
    assert ag["notify_mode"] == plr.PLR_NOTIFY_CHUNKS and ag["tile_bytes"] == 2048
    ag = pol("copy", "bf16", 8, (2 << 20) + 16, "packed", "packed")
    assert ag["notify_mode"] == plr.PLR_NOTIFY_CHECK and ag["tile_bytes"] == 4096
    half = pol("copy", "bf16", 8, 16 << 20, "scattered", "scattered")  # 2 MiB per source
    assert half["notify_mode"] == plr.PLR_NOTIFY_CHUNKS and half["tile_bytes"] == 2048
    agv = pol("copy", "bf16", 4, 6 << 20, "packed", "packed", part_bytes=[3 << 20, 1 << 20, 1 << 20, 1 << 20])
    assert agv["notify_mode"] == plr.PLR_NOTIFY_CHECK and agv["tile_bytes"] == 4096
    red = pol("reduce", "bf16", 8, 2 << 20, "packed", "packed")
    assert red["notify_mode"] == plr.PLR_NOTIFY_CHUNKS and red["tile_bytes"] == 8192  # decode-size share
    assert red["block"] == 512 and red["chunk_bytes"] == 16384
    small = pol("reduce", "bf16", 8, 512 << 10, "packed", "packed")  # at most 512 KiB: 4 KiB tiles
    assert small["tile_bytes"] == 4096 and small["block"] == 256 and small["chunk_bytes"] == 16384
    t64 = pol("reduce", "bf16", 8, 64 * 7168 * 2, "packed", "packed")
    assert t64["tile_bytes"] == 8192 and t64["block"] == 512
    # un-notified calls of a decode-size reduce keep 4 KiB tiles of 256 threads (no chunk
    # to wait for), 224 of them for [64, 7168] bf16; a caller's shape applies to both
    assert (t64["plain_tile_bytes"], t64["plain_block"], t64["plain_ntiles"]) == (4096, 256, 224)
    assert (small["plain_tile_bytes"], small["plain_block"], small["plain_ntiles"]) == (4096, 256, 128)
    tiny = pol("reduce", "bf16", 8, 48, "packed", "packed")  # one short tile
    assert (tiny["plain_tile_bytes"], tiny["plain_block"], tiny["plain_ntiles"]) == (48, 256, 1)
    for kw in (dict(tile_bytes=8192), dict(chunk_bytes=32768), dict(block=128)):
        o = pol("reduce", "bf16", 8, 64 * 7168 * 2, "packed", "packed", **kw)
        assert (o["plain_tile_bytes"], o["plain_block"]) == (o["tile_bytes"], o["block"]), kw
    lds = pol("reduce", "bf16", 8, 64 * 7168 * 2, "packed", "packed", datapath=plr.PLR_PATH_LDS)
    assert (lds["plain_tile_bytes"], lds["plain_block"]) == (lds["tile_bytes"], lds["block"])
    red = pol("reduce", "bf16", 8, 4 << 20, "packed", "packed")
    assert red["notify_mode"] == plr.PLR_NOTIFY_CHECK and red["tile_bytes"] == 2048
    assert (red["plain_tile_bytes"], red["plain_block"]) == (2048, 128)
    for L in (plr.plr_layout_create("copy", "bf16", 8, 2 << 20, "packed", "packed"),
              plr.plr_layout_create("allreduce", "bf16", 8, 1 << 20, "scattered", "scattered")):
        o = L.policy()
        assert (o["plain_tile_bytes"], o["plain_block"], o["plain_ntiles"]) == (o["tile_bytes"], o["block"], L.ntiles)


def test_tiles_and_chunks(plr):
    # a chunk is a whole number of tiles of one segment; ragged ends on both levels
    L = plr.plr_layout_create("reduce", "bf16", 2, 10 * 1024 + 32, "packed", "packed",
                              tile_bytes=1024, chunk_bytes=3000 // 16 * 16)
    p = L.policy()
    assert p["tile_bytes"] == 1024 and p["chunk_bytes"] == 3072
    assert L.ntiles == 11 and L.nchunks == 4
    C = plr.plr_layout_create("copy", "bf16", 4, 4 * 4096, "scattered", "transposed", tile_bytes=1024,
                              chunk_bytes=2048)
    assert C.ntiles == 16 * 4 and C.nchunks == 16 * 2
    T = plr.plr_layout_create("copy", "bf16", 2, 64, "packed", "packed", tile_bytes=1 << 20)
    assert T.policy()["tile_bytes"] == 64 and T.ntiles == 2 and T.nchunks == 2


def _code(fn, *a, **k):
    try:
        fn(*a, **k)
    except Exception as e:  # noqa: BLE001
        return getattr(e, "code", None)
    return 0


def test_layout_errors(plr):
    E = plr.PlrError
    mk = plr.plr_layout_create
    assert _code(mk, "reduce", "bf16", 0, 64, "packed", "packed") == plr.PLR_EINVAL
    assert _code(mk, "reduce", "bf16", 17, 64, "packed", "packed") == plr.PLR_EUNSUPPORTED
    assert _code(mk, "reduce", "bf16", 2, 40, "packed", "packed") == plr.PLR_EALIGN
    assert _code(mk, "reduce", "bf16", 3, 16 * 4, "scattered", "packed") == plr.PLR_EALIGN
    assert _code(mk, "reduce", "bf16", 3, 16 * 3, "scattered", "packed", rank=3) == plr.PLR_EINVAL
    assert _code(mk, "reduce", "bf16", 2, 64, "packed", "transposed") == plr.PLR_EINVAL
    assert _code(mk, "copy", "bf16", 2, 64, "packed", "transposed") == plr.PLR_EINVAL
    assert _code(mk, "copy", "bf16", 2, 64, "transposed", "packed") == plr.PLR_EINVAL
    assert _code(mk, "reduce", "bf16", 2, 64, "packed", "packed", mode=1) == plr.PLR_EUNSUPPORTED
    assert _code(mk, "reduce", "bf16", 2, 64, "packed", "packed", in_offsets=[0, 8]) == plr.PLR_EALIGN
    assert _code(mk, "reduce", "bf16", 2, 64, "packed", "packed", out_offsets=[0]) == plr.PLR_EINVAL
    assert _code(mk, "copy", "bf16", 2, 64, "packed", "packed", out_offsets=[0, 32]) == plr.PLR_EINVAL
    assert _code(mk, "copy", "bf16", 2, 64, "packed", "packed", out_offsets=[64, 0]) == 0
    assert _code(mk, "copy", "bf16", 9, 16 * 9, "scattered", "transposed",
                 in_offsets=list(range(0, 16 * 81, 16))) == plr.PLR_EUNSUPPORTED
    assert _code(mk, "copy", "bf16", 2, 64, "packed", "packed", chunk_bytes=24) == plr.PLR_EALIGN
    assert _code(mk, "copy", "bf16", 2, 64, "packed", "packed", block=100) == plr.PLR_EINVAL
    assert _code(mk, "copy", "bf16", 2, 64, "packed", "packed", unroll=3) == plr.PLR_EINVAL
    top = (1 << 64) - 16  # a segment that would end past 2^64 - 1
    assert _code(mk, "reduce", "bf16", 2, 64, "packed", "packed", in_offsets=[0, top]) == plr.PLR_EINVAL
    assert _code(mk, "copy", "bf16", 2, 64, "packed", "packed", in_offsets=[top, 0]) == plr.PLR_EINVAL
    assert _code(mk, "copy", "bf16", 2, 64, "packed", "packed", out_offsets=[0, top]) == plr.PLR_EINVAL
    assert issubclass(E, RuntimeError)


def test_layout_enum_fields_out_of_range(plr):
    """A C caller may store any int in the descriptor's enum fields: out-of-range values
    are PLR_EINVAL."""
    import ctypes

    for field, bad in [("op", -1), ("op", 3), ("dtype", 7), ("in_kind", -2), ("out_kind", 3)]:
        d = plr.plr_layout_desc()
        d.op, d.dtype, d.world, d.bytes_per_src = plr.PLR_OP_COPY, plr.PLR_BF16, 2, 64
        setattr(d, field, bad)
        h = ctypes.c_void_p()
        assert plr._lib.plr_layout_create(ctypes.byref(d), ctypes.byref(h)) == plr.PLR_EINVAL, field
        assert not h.value


def test_call_validation_without_device(plr):
    """Argument errors are caught on the host before any launch (fake addresses)."""
    L = plr.plr_layout_create("reduce", "bf16", 2, 4096, "packed", "packed")
    A, B, D = 1 << 40, (1 << 40) + (1 << 20), (1 << 40) + (2 << 20)
    assert _code(plr.plr_reduce, L, [A, B], D + 8) == plr.PLR_EALIGN
    assert _code(plr.plr_reduce, L, [A + 4, B], D) == plr.PLR_EALIGN
    assert _code(plr.plr_reduce, L, [A, B], A + 2048) == plr.PLR_EINVAL  # dst overlaps a source
    assert _code(plr.plr_reduce, L, [A, B], D, workspace=D + (1 << 20) + 8) == plr.PLR_EALIGN
    assert _code(plr.plr_copy, L, [A, B], D) == plr.PLR_EINVAL  # wrong op
    C = plr.plr_layout_create("copy", "bf16", 2, 4096, "packed", "packed")
    assert _code(plr.plr_copy, C, [A, B], A + 4096 - 16) == plr.PLR_EINVAL
    assert _code(plr.plr_notify, C, 2, D) == plr.PLR_EINVAL
    assert _code(plr.plr_notify, C, 0, D + 8) == plr.PLR_EALIGN
    cv = plr.plr_copy_v
    assert _code(cv, [A], [4], [D], 24, B, D, D, D) == plr.PLR_EALIGN
    assert _code(cv, [A] * 17, [1] * 17, [D] * 17, 16, B, D, D, D) == plr.PLR_EUNSUPPORTED
    assert _code(cv, [A + 8], [4], [D], 16, B, D, D, D) == plr.PLR_EALIGN
    assert _code(cv, [A], [4], [D], 16, A + 16, D, D, D) == plr.PLR_EINVAL  # dst overlaps source
    assert _code(cv, [A], [-1], [D], 16, B, D, D, D) == plr.PLR_EINVAL
    # row counts are bounded before they are summed: no signed overflow, no wrapped sizes
    big = (1 << 31) - 1
    assert _code(cv, [A, B], [big, 1], [D, D], 16, D, D, D, D) == plr.PLR_EUNSUPPORTED
    assert _code(cv, [A, B], [(1 << 62), (1 << 62)], [D, D], 16, D, D, D, D) == plr.PLR_EUNSUPPORTED
    assert _code(cv, [A] * 4, [(1 << 63) - 1] * 4, [D] * 4, 16, D, D, D, D) == plr.PLR_EUNSUPPORTED
    # an output of 2^64 bytes or more cannot exist; its size would wrap the overlap check
    assert _code(cv, [A], [2], [D], 1 << 63, 1 << 40, D, D, D) == plr.PLR_EINVAL


def test_scratch_bytes(plr):
    # header + one key per row + (segments x W) counts + (segments x 16) segment rows,
    # int32 each, every region rounded up to 256 bytes
    assert plr.plr_copy_v_scratch_bytes(8, [4096] * 8) == 256 + 8 * 4096 * 4 + 32 * 8 * 4 + 32 * 16 * 4
    assert plr.plr_copy_v_scratch_bytes(2, [1, 2]) == 256 + 256 + 256 + 256
    assert plr.plr_copy_v_scratch_bytes(2, [1025, 0]) == 256 + 4352 + 256 + 256
    assert plr.plr_copy_v_scratch_bytes(2, [-1, 0]) == 0
    assert plr.plr_copy_v_scratch_bytes(0, []) == 0
    assert plr.plr_copy_v_scratch_bytes(2, [(1 << 31) - 1, 1]) == 0  # more than 2^31 - 1 rows
    assert plr.plr_copy_v_scratch_bytes(4, [(1 << 62)] * 4) == 0  # the sum would wrap
    assert plr.plr_copy_v_scratch_bytes(1, [(1 << 31) - 1]) > 8 << 30


def test_strerror(plr):
    for code in range(7):
        assert plr.plr_strerror(code) != "unknown error"
    assert "timed out" in plr.plr_strerror(plr.PLR_ETIMEOUT)
    assert "scratch" in plr.plr_strerror(plr.PLR_ETOOLARGE)
    assert plr.plr_version().startswith("plr")


def test_lds_datapath_layouts(plr):
    L = plr.plr_layout_create("reduce", "bf16", 8, 1 << 20, "packed", "packed", datapath=plr.PLR_PATH_LDS)
    p = L.policy()
    assert p["datapath"] == plr.PLR_PATH_LDS and p["block"] == 256 and p["tile_bytes"] % 4096 == 0
    C = plr.plr_layout_create("copy", "bf16", 4, 1 << 16, "packed", "packed", datapath=plr.PLR_PATH_LDS)
    assert C.policy()["block"] == 256
    # a single short tile is fine; several tiles must be whole 4 KiB slabs
    plr.plr_layout_create("reduce", "bf16", 2, 1024, "packed", "packed", datapath=plr.PLR_PATH_LDS)
    assert _code(plr.plr_layout_create, "reduce", "bf16", 2, 16384, "packed", "packed",
                 datapath=plr.PLR_PATH_LDS, tile_bytes=2048) == plr.PLR_EINVAL
    assert _code(plr.plr_layout_create, "reduce", "bf16", 2, 16384, "packed", "packed",
                 datapath=plr.PLR_PATH_LDS, block=128) == plr.PLR_EINVAL


def test_allreduce_layouts(plr):
    L = plr.plr_layout_create("allreduce", "bf16", 8, 16 * 8 * 100, "scattered", "scattered")
    assert L.policy()["datapath"] == plr.PLR_PATH_DIRECT and L.dst_bytes == 16 * 8 * 100
    C = plr.plr_layout_create("allreduce", "bf16", 4, 4 * 64 * 1024 * 3, "scattered", "scattered",
                              datapath=plr.PLR_PATH_COMPOSED, tile_bytes=64 * 1024)
    assert C.policy()["tile_bytes"] == 64 * 1024 and C.ntiles == 4 * 3 and C.nchunks == 12
    assert C.workspace_bytes == 256 + 12 * 8
    # the composed policy: as few tiles as keep all ntiles + 16 (the gather lag)
    # workgroups of a call resident at once on 256 CUs, i.e. at most (256 - 16) / W
    # tiles per slice: the smallest such tile in whole workgroup steps (256 threads x
    # 16 bytes), or in 16-byte vectors when a tile is shorter than one step
    for W, S in [(4, 4 * 64 * 1024 * 3), (8, 8192 * 7168 * 2), (2, 1 << 24), (16, 16 * 16 * 1000), (3, 48 * 1000)]:
        P = plr.plr_layout_create("allreduce", "bf16", W, S, "scattered", "scattered",
                                  datapath=plr.PLR_PATH_COMPOSED)
        tile, slice_ = P.policy()["tile_bytes"], S // W
        tps = -(-slice_ // tile)
        g = 4096 if tile >= 4096 else 16
        assert tile % g == 0 and P.ntiles == W * tps and P.ntiles + 16 <= 256, (W, S, tile)
        per_slice = (256 - 16) // W
        assert tps <= per_slice and (tile == g or -(-slice_ // (tile - g)) > per_slice), (W, S, tile)
        assert P.workspace_bytes == 256 + P.ntiles * 8
    assert plr.plr_layout_create("allreduce", "bf16", 8, 8192 * 7168 * 2, "scattered", "scattered",
                                 datapath=plr.PLR_PATH_COMPOSED).ntiles == 240
    mk = plr.plr_layout_create
    # a caller's tile size whose ntiles + 16 workgroups would not all be resident at once
    # on 256 CUs is refused for the composed path (the fused path takes any tile size)
    assert _code(mk, "allreduce", "bf16", 8, 8 * 30 * 1024, "scattered", "scattered",
                 datapath=plr.PLR_PATH_COMPOSED, tile_bytes=1024) == 0  # 240 tiles + 16
    assert _code(mk, "allreduce", "bf16", 8, 8 * 31 * 1024, "scattered", "scattered",
                 datapath=plr.PLR_PATH_COMPOSED, tile_bytes=1024) == plr.PLR_EUNSUPPORTED  # 248 + 16
    assert _code(mk, "allreduce", "bf16", 8, 8 * 31 * 1024, "scattered", "scattered", tile_bytes=1024) == 0
    assert _code(mk, "allreduce", "bf16", 4, 64, "packed", "packed") == plr.PLR_EINVAL
    assert _code(mk, "allreduce", "bf16", 3, 16 * 4, "scattered", "scattered") == plr.PLR_EALIGN
    assert _code(mk, "allreduce", "bf16", 2, 64, "scattered", "scattered", datapath=plr.PLR_PATH_LDS) == plr.PLR_EINVAL
    assert _code(mk, "reduce", "bf16", 2, 64, "packed", "packed", datapath=plr.PLR_PATH_COMPOSED) == plr.PLR_EINVAL
    A, B = 1 << 40, (1 << 40) + (1 << 24)
    assert _code(plr.plr_allreduce, C, [A + 16 * k for k in range(4)], [B] * 4) in (plr.PLR_EINVAL, plr.PLR_EALIGN)
    assert _code(plr.plr_allreduce, C, [A + (1 << 20) * k for k in range(4)],
                 [B + (1 << 20) * k for k in range(4)]) == plr.PLR_EINVAL  # composed needs a workspace
    assert _code(plr.plr_notify, C, 0, B) == plr.PLR_EINVAL


def test_packet_layouts_and_validation(plr):
    L = plr.plr_layout_create("reduce", "bf16", 4, 4 * 4096, "scattered", "packed", rank=1)
    assert L.packet_bytes == 4 * 4096  # two slots of 2 x the 4096-byte share
    C = plr.plr_layout_create("copy", "bf16", 2, 4096, "packed", "packed")
    assert C.packet_bytes == 0
    A, P, D, WS = 1 << 40, (1 << 40) + (1 << 24), (1 << 40) + (2 << 24), (1 << 40) + (3 << 24)
    pk = [P + k * L.packet_bytes for k in range(4)]
    src = [A + k * (1 << 20) for k in range(4)]
    assert _code(plr.plr_pack, C, 0, src[:2], pk[:2]) == plr.PLR_EINVAL  # copy layouts have no packets
    assert _code(plr.plr_pack, L, 4, src, pk) == plr.PLR_EINVAL  # no source 4
    assert _code(plr.plr_pack, L, -2, src, pk) == plr.PLR_EINVAL
    assert _code(plr.plr_pack, L, 0, [A + 8] + src[1:], pk) == plr.PLR_EALIGN
    assert _code(plr.plr_pack, L, -1, src[:3] + [A + 8], pk) == plr.PLR_EALIGN
    # source 1's share of a scattered layout at rank 1 starts 4096 bytes into its buffer
    assert _code(plr.plr_pack, L, 1, src, pk[:1] + [src[1] + 4096 + 16] + pk[2:]) == plr.PLR_EINVAL
    assert _code(plr.plr_pack, L, -1, src, pk[:3] + [pk[2] + 4096]) == plr.PLR_EINVAL  # packets overlap
    assert _code(plr.plr_pack, L, -1, src, pk[:3] + [pk[2] + 12288]) == plr.PLR_EINVAL  # in the second slot
    assert _code(plr.plr_reduce_packets, L, pk, D, 0) == plr.PLR_EINVAL  # workspace required
    assert _code(plr.plr_reduce_packets, L, pk, D, WS + 8) == plr.PLR_EALIGN
    assert _code(plr.plr_reduce_packets, L, pk, pk[2] + 16, WS) == plr.PLR_EINVAL  # dst inside packets
    assert _code(plr.plr_reduce_packets, L, pk[:3] + [pk[3] + 4], D, WS) == plr.PLR_EALIGN
    assert L.epoch == 0  # rejected calls do not advance the epoch


def test_timing_events_arguments(plr):
    """Only a full pair (or none) of measurement events is accepted; nothing is launched."""
    lib = plr._lib
    assert lib.plr_set_timing_events(ctypes.c_void_p(0x1000), None) == plr.PLR_EINVAL
    assert lib.plr_set_timing_events(None, ctypes.c_void_p(0x1000)) == plr.PLR_EINVAL
    assert lib.plr_set_timing_events(None, None) == plr.PLR_OK


def test_variable_length_layouts(plr, oracle_mod):
    """AllGatherV and ReduceScatterV layouts (part_bytes): segments follow the oracle's
    prefix-sum offsets, every segment has its own tile and chunk count, and the flags
    of a source are its own chunks."""
    import synth

    W, T = 8, 1 << 20
    parts = synth.zipf_split(T, W)
    offs = oracle_mod.part_offsets(parts)
    G = plr.plr_layout_create("copy", "bf16", W, T, "packed", "packed", part_bytes=parts,
                              tile_bytes=2048, chunk_bytes=8192)
    assert G.segments() == [(w, 0, offs[w], parts[w]) for w in range(W)]
    assert G.dst_bytes == T
    tiles = [-(-p // 2048) for p in parts]
    assert G.ntiles == sum(tiles)
    assert G.nchunks == sum(-(-t // 4) for t in tiles)
    assert G.workspace_bytes == 256 + 2 * G.nchunks * 8
    for r in (0, 3, 7):
        R = plr.plr_layout_create("reduce", "f16", W, T, "scattered", "packed", rank=r, part_bytes=parts)
        assert R.segments() == [(w, offs[r], 0, parts[r]) for w in range(W)]
        assert R.dst_bytes == parts[r]
    # empty partitions: an empty share, and an AllGatherV segment with no tiles
    Z = plr.plr_layout_create("copy", "bf16", 3, 64, "packed", "packed", part_bytes=[32, 0, 32], tile_bytes=16)
    assert Z.segments() == [(0, 0, 0, 32), (1, 0, 32, 0), (2, 0, 32, 32)] and Z.ntiles == 4
    E = plr.plr_layout_create("reduce", "bf16", 3, 64, "scattered", "packed", rank=1, part_bytes=[32, 0, 32])
    assert E.dst_bytes == 0 and E.ntiles == 0
    # errors
    bad = plr.plr_layout_create
    assert _code(bad, "copy", "bf16", 2, 64, "packed", "packed", part_bytes=[32, 16]) == plr.PLR_EINVAL  # sum
    # sizes whose 64-bit sum wraps around to T are still past T
    wrap = [1 << 63, 1 << 63, 16]
    assert _code(bad, "reduce", "bf16", 3, 16, "scattered", "packed", rank=2, part_bytes=wrap) == plr.PLR_EINVAL
    assert _code(bad, "copy", "bf16", 3, 16, "packed", "packed", part_bytes=wrap) == plr.PLR_EINVAL
    assert _code(bad, "copy", "bf16", 2, 64, "packed", "packed", part_bytes=[40, 24]) == plr.PLR_EALIGN
    assert _code(bad, "copy", "bf16", 2, 64, "scattered", "transposed", part_bytes=[32, 32]) == plr.PLR_EINVAL
    assert _code(bad, "reduce", "bf16", 2, 64, "packed", "packed", part_bytes=[32, 32]) == plr.PLR_EINVAL
    assert _code(bad, "allreduce", "bf16", 2, 64, "scattered", "scattered", part_bytes=[32, 32]) == plr.PLR_EINVAL
    assert _code(bad, "copy", "bf16", 2, 8192, "packed", "packed", part_bytes=[4096, 4096],
                 datapath=plr.PLR_PATH_LDS) == plr.PLR_EUNSUPPORTED


def test_atom_header_standalone(tmp_path):
    """include/plr_atom.h compiles on its own for gfx950 (only plr.h beside it) and the
    user-kernel library the GPU tests load exports its launchers."""
    src = tmp_path / "user.hip"
    src.write_text('#include "plr_atom.h"\n'
                   "__global__ void k(void* d, const void* s, size_t n) {\n"
                   "  plr::atom::Atom<256, 2>::copy(d, s, n);\n"
                   "  const void* srcs[2] = {s, s};\n"
                   "  plr::atom::Atom<256>::reduce<PLR_BF16, 2>(d, srcs, n);\n}\n")
    r = subprocess.run(["/opt/rocm/bin/hipcc", "-x", "hip", "--offload-arch=gfx950", "--cuda-device-only",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-std=c++17", "-O3",
                        "-I", os.path.join(ROOT, "include"), "-c", str(src), "-o", str(tmp_path / "user.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lib = os.path.join(ROOT, "tests", "libatom_kernels.so")
    if os.path.exists(lib):
        out = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True).stdout
        assert {"atom_block_copy", "atom_block_reduce", "atom_pipeline"} <= set(re.findall(r" T (atom_\w+)", out))


def test_one_hip_runtime_whatever_the_import_order(plr):
    """Importing the binding before torch must still leave a single HIP runtime in the
    process (torch's), so that the library launches on the runtime that owns torch's
    memory and streams."""
    code = ("import reduce_atom_amd, torch\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "print(sorted({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    out = subprocess.run([os.sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    paths = eval(out.stdout.strip().splitlines()[-1])
    assert len(paths) == 1, paths


def test_reduce_unroll_fits_the_registers(plr):
    """A reduce lane holds unroll x W vectors: four per source is kept up to W = 14 and
    becomes two from W = 15 (4 x 15 vectors would spill)."""
    for W, want in [(1, 4), (8, 4), (14, 4), (15, 2), (16, 2)]:
        L = plr.plr_layout_create("reduce", "bf16", W, 16 * W * 64, "packed", "packed", unroll=4)
        assert L.policy()["unroll"] == want, W
    C = plr.plr_layout_create("copy", "bf16", 16, 16 * 64, "packed", "packed", unroll=4)
    assert C.policy()["unroll"] == 4


def test_copy_v_scatter_covers_every_tile(tmp_path):
    """The row scatter's run-to-workgroup mapping (reduce_atom_amd/csrc/copy_v_grid.h, the
    functions its launcher and kernel use) moves every tile exactly once, also when the
    column cap makes columns stride and in the small form, whose last column moves no
    tile. Built and run on the host with a lowered cap."""
    exe = tmp_path / "cv_grid_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror",
                    "-I", os.path.join(ROOT, "reduce_atom_amd", "csrc"),
                    os.path.join(ROOT, "tests", "host", "cv_grid_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")


def test_binding_checks_list_lengths(plr):
    """The binding refuses lists whose length differs from what the C side reads (it
    would read past a short array and hand the kernels garbage addresses), and
    destination tensors that are not int32. Integer addresses: nothing is launched."""
    import torch

    L = plr.plr_layout_create("reduce", "bf16", 4, 4096, "packed", "packed")
    with pytest.raises(ValueError, match="srcs"):
        plr.plr_reduce(L, [16, 32, 48], 4096 * 16)
    C = plr.plr_layout_create("copy", "bf16", 4, 4096, "packed", "packed")
    with pytest.raises(ValueError, match="srcs"):
        plr.plr_copy(C, [16] * 5, 1 << 20)
    A = plr.plr_layout_create("allreduce", "bf16", 2, 4096, "scattered", "scattered")
    with pytest.raises(ValueError, match="dsts"):
        plr.plr_allreduce(A, [16, 32], [64])
    with pytest.raises(ValueError, match="packets"):
        plr.plr_reduce_packets(L, [16], 1 << 20, 1 << 21)
    with pytest.raises(ValueError, match="in_offsets"):
        plr.plr_layout_create("reduce", "bf16", 4, 4096, "packed", "packed", in_offsets=[0, 0, 0])
    with pytest.raises(ValueError, match="out_offsets"):
        plr.plr_layout_create("copy", "bf16", 2, 4096, "scattered", "transposed", out_offsets=[0, 0])
    with pytest.raises(ValueError, match="part_bytes"):
        plr.plr_layout_create("copy", "bf16", 3, 4096, "packed", "packed", part_bytes=[2048, 2048])
    with pytest.raises(ValueError, match="rows_per_src"):
        plr.plr_copy_v([16, 32], [4], [64, 80], 64, 1 << 20, 1 << 21, 1 << 22, 1 << 23)
    with pytest.raises(ValueError, match="dest_of_row"):
        plr.plr_copy_v([16, 32], [4, 4], [64], 64, 1 << 20, 1 << 21, 1 << 22, 1 << 23)
    with pytest.raises(ValueError, match="int32"):
        plr.plr_copy_v([16], [4], [torch.zeros(4, dtype=torch.int64)], 64, 1 << 20, 1 << 21, 1 << 22, 1 << 23)
    with pytest.raises(ValueError, match="rows_per_src"):
        plr.plr_copy_v_scratch_bytes(3, [1, 2])


def test_copy_v_noalloc_limits_without_device(plr):
    """The allocation-free copy_v: its fixed scratch size, and requests beyond it (or
    with invalid row counts) rejected on the host before any device call."""
    cap = plr.plr_copy_v_noalloc_max_scratch_bytes()
    assert cap == 4 << 20
    lib = ctypes.CDLL(plr.LIB_PATH)
    fn = lib.plr_copy_v_noalloc
    fn.restype = ctypes.c_int
    vp = ctypes.c_void_p
    fn.argtypes = [ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(vp),
                   ctypes.c_size_t, vp, vp, vp, vp]
    ptrs = (vp * 2)(16, 32)

    def call(rows):
        r = (ctypes.c_int64 * 2)(*rows)
        return fn(2, ptrs, r, ptrs, 64, 1 << 30, 1 << 31, 1 << 32, None)

    too_many = cap // 4  # one key of 4 bytes per row alone fills the scratch
    assert plr.plr_copy_v_scratch_bytes(2, [too_many, 0]) > cap
    assert call([too_many, 0]) == plr.PLR_ETOOLARGE
    assert call([-1, 4]) == plr.PLR_EINVAL
    assert call([1 << 62, 1 << 62]) == plr.PLR_EUNSUPPORTED  # as plr_copy_v, not a wrapped size
    assert fn(0, ptrs, (ctypes.c_int64 * 2)(1, 1), ptrs, 64, 1, 2, 3, None) == plr.PLR_EINVAL
    assert fn(17, ptrs, (ctypes.c_int64 * 2)(1, 1), ptrs, 64, 1, 2, 3, None) == plr.PLR_EUNSUPPORTED


def test_layout_queries_on_null(plr):
    """Every query on a NULL layout returns its documented error value, not a crash."""
    lib = plr._lib
    assert lib.plr_layout_policy(None, None, None, None, None, None, None, None, None) == plr.PLR_EINVAL
    assert lib.plr_layout_plain_shape(None, None, None, None) == plr.PLR_EINVAL
    assert lib.plr_layout_ntiles(None) == -1 and lib.plr_layout_nchunks(None) == -1
    assert lib.plr_layout_nsegments(None) == -1
    assert lib.plr_layout_workspace_bytes(None) == 0 and lib.plr_layout_dst_bytes(None) == 0
    assert lib.plr_layout_packet_bytes(None) == 0 and lib.plr_layout_epoch(None) == 0
    L = plr.plr_layout_create("reduce", "bf16", 2, 4096, "packed", "packed")
    assert lib.plr_layout_plain_shape(L.handle, None, None, None) == plr.PLR_OK  # outputs may be NULL


def test_resident_workgroup_cap(plr):
    """Resident workgroups per CU are capped through an LDS reservation (leaving 512 bytes
    for the kernel's own): the policy caps the fused AllReduce of more than 2 MiB per source
    at 8 and nothing else; callers may cap any direct-path layout; the LDS-staged and
    composed paths never are capped; bad values are refused."""
    def occ(*a, **k):
        p = plr.plr_layout_create(*a, **k).policy()
        return p["wgs_per_cu"], p["lds_reserve"]
    big = ("reduce", "bf16", 8, 8192 * 7168 * 2, "packed", "packed")
    assert occ(*big) == (0, 0)
    assert occ(*big, wgs_per_cu=-1) == (0, 0)
    assert occ(*big, wgs_per_cu=5) == (5, 32256)
    for k in (1, 2, 3, 4, 6, 8, 16):
        cap, lds = occ(*big, wgs_per_cu=k)
        assert cap == k and 163840 // ((lds + 256 + 511) // 512 * 512) == k
    assert occ("reduce", "bf16", 8, 2 << 20, "packed", "packed") == (0, 0)  # decode-size share
    assert occ("reduce", "bf16", 8, 4 << 20, "scattered", "packed", rank=1) == (0, 0)  # 512 KiB per source
    assert occ("copy", "bf16", 8, 64 << 20, "packed", "packed") == (0, 0)
    assert occ("copy", "bf16", 8, 64 << 20, "packed", "packed", wgs_per_cu=8)[0] == 8
    assert occ("allreduce", "bf16", 8, 1 << 24, "scattered", "scattered") == (8, 19968)
    assert occ("allreduce", "bf16", 8, 2 << 20, "scattered", "scattered") == (0, 0)  # 2 MiB: uncapped
    assert occ("allreduce", "bf16", 8, 1 << 24, "scattered", "scattered", wgs_per_cu=3) == (3, 53760)
    assert occ("allreduce", "bf16", 8, 1 << 24, "scattered", "scattered", wgs_per_cu=-1) == (0, 0)
    assert occ("allreduce", "bf16", 8, 1 << 24, "scattered", "scattered", wgs_per_cu=4)[0] == 4
    assert occ(*big, datapath=plr.PLR_PATH_LDS) == (0, 0)
    assert occ(*big, datapath=plr.PLR_PATH_LDS, wgs_per_cu=4) == (0, 0)
    assert occ("allreduce", "bf16", 8, 1 << 24, "scattered", "scattered", datapath=plr.PLR_PATH_COMPOSED,
               wgs_per_cu=4) == (0, 0)
    for bad in (17, -2, 1000):
        assert _code(plr.plr_layout_create, *big, wgs_per_cu=bad) == plr.PLR_EINVAL



def test_binding_rejects_tensors_smaller_than_the_call_uses(plr):
    """The C side takes bare pointers; the binding checks every tensor argument against
    the bytes the call reads or writes through it before anything reaches the library
    (CPU tensors here: a call whose sizes pass stops at the device check instead)."""
    import torch

    W, n = 4, 2048
    L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed")
    ok = [torch.empty(n, dtype=torch.bfloat16) for _ in range(W)]
    short = ok[:3] + [torch.empty(n - 8, dtype=torch.bfloat16)]
    with pytest.raises(ValueError, match=r"srcs\[3\]: 4080 bytes, the call uses 4096"):
        plr.plr_reduce(L, short, torch.empty(n, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match=r"dst: 4094 bytes"):
        plr.plr_reduce(L, ok, torch.empty(n - 1, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match=r"workspace: 8 bytes"):
        plr.plr_reduce(L, ok, torch.empty(n, dtype=torch.bfloat16), torch.empty(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="device tensor expected"):
        plr.plr_reduce(L, ok, torch.empty(n, dtype=torch.bfloat16))
    # explicit offsets: a source must reach its segment's end
    Lo = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed", in_offsets=[0, 0, 0, 4096])
    assert Lo.src_extent() == [4096, 4096, 4096, 8192]
    with pytest.raises(ValueError, match=r"srcs\[3\]: 4096 bytes, the call uses 8192"):
        plr.plr_reduce(Lo, ok, torch.empty(n, dtype=torch.bfloat16))
    # AllToAll: every source, the whole transposed output
    A = plr.plr_layout_create("copy", "bf16", W, 4096, "scattered", "transposed")
    c_ok = [torch.empty(4096, dtype=torch.uint8) for _ in range(W)]
    with pytest.raises(ValueError, match=r"dst: 16383 bytes, the call uses 16384"):
        plr.plr_copy(A, c_ok, torch.empty(W * 4096 - 1, dtype=torch.uint8))
    # variable-length AllToAll: rows, destinations, output, counts and scratch
    rows, rb = [3, 0, 5, 1], 64
    srcs = [torch.empty(r * rb, dtype=torch.uint8) for r in rows]
    dest = [torch.zeros(r, dtype=torch.int32) for r in rows]
    args = dict(row_bytes=rb, dst=torch.empty(9 * rb, dtype=torch.uint8), counts=torch.empty(16, dtype=torch.int64),
                offsets=torch.empty(16, dtype=torch.int64),
                scratch=torch.empty(plr.plr_copy_v_scratch_bytes(W, rows), dtype=torch.uint8))
    bad_dest = dest[:2] + [torch.zeros(4, dtype=torch.int32)] + dest[3:]
    with pytest.raises(ValueError, match=r"dest_of_row\[2\]: 16 bytes, the call uses 20"):
        plr.plr_copy_v(srcs, rows, bad_dest, **args)
    with pytest.raises(ValueError, match=r"dst: 512 bytes, the call uses 576"):
        plr.plr_copy_v(srcs, rows, dest, **{**args, "dst": torch.empty(8 * rb, dtype=torch.uint8)})
    with pytest.raises(ValueError, match=r"counts: 120 bytes"):
        plr.plr_copy_v(srcs, rows, dest, **{**args, "counts": torch.empty(15, dtype=torch.int64)})
    with pytest.raises(ValueError, match=r"scratch: 8 bytes"):
        plr.plr_copy_v(srcs, rows, dest, **{**args, "scratch": torch.empty(8, dtype=torch.uint8)})
    with pytest.raises(ValueError, match="device tensor expected"):
        plr.plr_copy_v(srcs, rows, dest, **args)
