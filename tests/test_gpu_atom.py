"""User kernels built on the device-callable Atom (include/plr_atom.h; Purlin README
"Device-side": a kernel calls the Atom's copy or reduce on its own slice), checked
against the oracle: per-workgroup copies, ordered reductions with and without a fused
residual-add epilogue, stage / notify / consume inside one kernel, and producer kernels
that announce their own chunks (flags or packets) to the library's consumers."""
import ctypes
import os

import numpy as np
import pytest
import torch

import synth
from plrtest import assert_same, from_dev, to_dev

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
DTYPES = {"bf16": 0, "f16": 1, "f32": 2}


@pytest.fixture(scope="module")
def atom():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import reduce_atom_amd  # noqa: F401  (the GPU tests run with the library built)

    lib = ctypes.CDLL(os.path.join(HERE, "libatom_kernels.so"))
    vp, sz, i, u, ull = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint, ctypes.c_ulonglong
    lib.atom_block_copy.argtypes = [vp, vp, sz, u, i, vp]
    lib.atom_block_reduce.argtypes = [i, i, ctypes.POINTER(vp), vp, vp, sz, u, i, vp]
    lib.atom_pipeline.argtypes = [vp, vp, vp, sz, u, u, vp, ull, ull, ull, vp, vp]
    lib.atom_produce.argtypes = [i, i, ctypes.POINTER(vp), ctypes.POINTER(vp), sz, sz, vp, ull, vp]
    return lib


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("threads", [64, 128, 256, 512])
@pytest.mark.parametrize("per_block", [16, 2048, 4096 + 48])
def test_block_copy(atom, oracle_mod, threads, per_block):
    nblocks = 37
    total = nblocks * per_block
    src_np = synth.bits_np(41, 9, 0, total + 16)
    src = to_dev(src_np)
    dst = torch.full((total + 16,), 0x5A, dtype=torch.uint8, device="cuda")
    assert atom.atom_block_copy(dst.data_ptr(), src.data_ptr(), per_block, nblocks, threads, _stream()) == 0
    torch.cuda.synchronize()
    got = from_dev(dst)
    assert np.array_equal(got[:total], oracle_mod.copy([src_np], [(0, 0, 0, total)], total))
    assert (got[total:] == 0x5A).all()  # nothing past the last block


@pytest.mark.parametrize("dtype", list(DTYPES))
@pytest.mark.parametrize("W", [1, 2, 3, 8])
@pytest.mark.parametrize("unroll", [1, 2])
@pytest.mark.parametrize("residual", [False, True])
def test_block_reduce(atom, oracle_mod, dtype, W, unroll, residual):
    """Slices of 2 KiB + 16 B per workgroup (a ragged step for 128 threads); with the
    residual epilogue the result is the ordered reduction with the residual appended
    as the last source (one binary32 accumulator, one rounding)."""
    eb = oracle_mod.ELEM_BYTES[dtype]
    per_block, nblocks = 2048 + 16, 9
    total = per_block * nblocks
    srcs_np = [synth.normal_np(42, 9, w, total // eb, dtype=dtype) for w in range(W)]
    res_np = synth.normal_np(42, 9, 99, total // eb, dtype=dtype)
    srcs = [to_dev(s) for s in srcs_np]
    res = to_dev(res_np)
    dst = torch.full((total,), 0x5A, dtype=torch.uint8, device="cuda")
    ptrs = (ctypes.c_void_p * W)(*[s.data_ptr() for s in srcs])
    rc = atom.atom_block_reduce(DTYPES[dtype], W, ptrs, res.data_ptr() if residual else None, dst.data_ptr(),
                                per_block, nblocks, unroll, _stream())
    assert rc == 0
    torch.cuda.synchronize()
    ref = oracle_mod.reduce(dtype, srcs_np + ([res_np] if residual else []))
    assert_same(dtype, from_dev(dst), ref.view(np.uint8))


def test_pipeline_in_one_kernel(atom, oracle_mod):
    """64 chunks staged into `mid`, each announced by its flag, consumed 4 workgroups
    later into `dst`; three epochs on the same flags without a reset."""
    nchunks, lag, chunk = 64, 4, 4096 + 16
    total = nchunks * chunk
    src_np = synth.bits_np(43, 9, 0, total)
    src = to_dev(src_np)
    mid = torch.empty(total, dtype=torch.uint8, device="cuda")
    flags = torch.zeros(nchunks, dtype=torch.int64, device="cuda")
    err = torch.zeros(4, dtype=torch.int32, device="cuda")
    for epoch in (1, 2, 3):
        dst = torch.full((total,), 0x5A, dtype=torch.uint8, device="cuda")
        rc = atom.atom_pipeline(src.data_ptr(), mid.data_ptr(), dst.data_ptr(), chunk, nchunks, lag,
                                flags.data_ptr(), epoch, epoch, 1 << 22, err.data_ptr(), _stream())
        assert rc == 0
        torch.cuda.synchronize()
        assert int(err[0].item()) == 0
        assert np.array_equal(from_dev(dst), oracle_mod.copy([src_np], [(0, 0, 0, total)], total)), epoch
        assert (flags.cpu().numpy() == epoch).all()


def test_pipeline_bounded_wait_gives_up(atom):
    """Producers that announce a stale epoch: every consumer's bounded wait gives up,
    records the error and copies nothing (no hang)."""
    nchunks, lag, chunk = 16, 2, 1024
    src = torch.ones(nchunks * chunk, dtype=torch.uint8, device="cuda")
    mid = torch.empty_like(src)
    dst = torch.zeros_like(src)
    flags = torch.zeros(nchunks, dtype=torch.int64, device="cuda")
    err = torch.zeros(4, dtype=torch.int32, device="cuda")
    assert atom.atom_pipeline(src.data_ptr(), mid.data_ptr(), dst.data_ptr(), chunk, nchunks, lag,
                              flags.data_ptr(), 1, 2, 2000, err.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    assert int(err[0].item()) == 1
    assert int(dst.sum().item()) == 0
    assert (flags.cpu().numpy() == 1).all()


def _produce(atom, mode, ins, outs, share, chunk, flags_ptr, epoch, stream=None):
    W = len(ins)
    vp = ctypes.c_void_p
    rc = atom.atom_produce(mode, W, (vp * W)(*[t.data_ptr() for t in ins]), (vp * W)(*[t.data_ptr() for t in outs]),
                           share, chunk, flags_ptr, epoch, stream if stream is not None else _stream())
    assert rc == 0


def _producer_setup(L, mode, share):
    """The producer's chunks are the layout's flags; packet buffers are the layout's size."""
    chunk = L.policy()["chunk_bytes"]
    assert (share + chunk - 1) // chunk == L.nchunks
    ws = torch.zeros(max(L.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
    W = L.world
    if mode == "flags":
        outs = [torch.empty(share, dtype=torch.uint8, device="cuda") for _ in range(W)]
    else:
        outs = [torch.zeros(L.packet_bytes, dtype=torch.uint8, device="cuda") for _ in range(W)]
    return chunk, ws, outs


@pytest.mark.parametrize("mode", ["flags", "packets"])
@pytest.mark.parametrize("T", [1, 37, 64])
def test_producer_kernel_feeds_the_library_consumer(atom, oracle_mod, T, mode):
    """A user producer that announces its own chunks (section 3.2, Figure 7): plain stores
    plus signal_flag on the layout's workspace flags, consumed by the notified plr_reduce;
    or packets written with store_packet, consumed by plr_reduce_packets. Three epochs on
    one workspace and one set of packet buffers (both slots), each against the oracle."""
    import reduce_atom_amd as plr

    W, n = 8, T * 7168
    share = 2 * n
    L = plr.plr_layout_create("reduce", "bf16", W, share, "packed", "packed")
    chunk, ws, outs = _producer_setup(L, mode, share)
    for e in range(3):
        ins_np = [synth.normal_np(50 + e, 13, w, n, 1.0) for w in range(W)]
        ins = [to_dev(x) for x in ins_np]
        epoch = L.epoch + 1
        _produce(atom, 1 if mode == "flags" else 2, ins, outs, share, chunk, ws.data_ptr() + 256, epoch)
        dst = torch.full((share,), 0x5A, dtype=torch.uint8, device="cuda")
        if mode == "flags":
            plr.plr_reduce(L, outs, dst, ws)
        else:
            plr.plr_reduce_packets(L, outs, dst, ws)
        torch.cuda.synchronize()
        assert plr.plr_check(L, ws) == plr.PLR_OK
        assert L.epoch == epoch
        assert_same("bf16", from_dev(dst), oracle_mod.reduce("bf16", ins_np).view(np.uint8),
                    f"T={T} {mode} epoch {epoch}")


@pytest.mark.parametrize("mode", ["flags", "packets"])
def test_producer_kernel_beside_a_waiting_consumer(atom, oracle_mod, mode):
    """The producer kernel queued on one stream behind a sleep, the consumer on another
    (queued second: a consumer queued first on a hardware queue it shares with the producer
    could only time out): where the streams overlap the consumer reaches the chunks before
    they are announced, and it reads every chunk only once it is."""
    import reduce_atom_amd as plr

    W, T = 8, 8
    n = T * 7168
    share = 2 * n
    L = plr.plr_layout_create("reduce", "bf16", W, share, "packed", "packed", spin_limit=1 << 22)
    chunk, ws, outs = _producer_setup(L, mode, share)
    for e in range(3):
        ins_np = [synth.normal_np(60 + e, 14, w, n, 1.0) for w in range(W)]
        ins = [to_dev(x) for x in ins_np]
        torch.cuda.synchronize()
        epoch = L.epoch + 1
        dst = torch.full((share,), 0x5A, dtype=torch.uint8, device="cuda")
        producer, consumer = torch.cuda.Stream(), torch.cuda.Stream()
        with torch.cuda.stream(producer):
            if hasattr(torch.cuda, "_sleep"):
                torch.cuda._sleep(20_000_000)
            _produce(atom, 1 if mode == "flags" else 2, ins, outs, share, chunk, ws.data_ptr() + 256, epoch)
        with torch.cuda.stream(consumer):
            if mode == "flags":
                plr.plr_reduce(L, outs, dst, ws)
            else:
                plr.plr_reduce_packets(L, outs, dst, ws)
        torch.cuda.synchronize()
        assert plr.plr_check(L, ws) == plr.PLR_OK
        assert_same("bf16", from_dev(dst), oracle_mod.reduce("bf16", ins_np).view(np.uint8),
                    f"{mode} epoch {epoch}")
