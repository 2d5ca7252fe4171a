"""Seeded synthetic inputs shared by the tests, the oracle checks and the benchmark.

This module draws random numbers and shapes them into the workloads' value
distributions. It holds none of the datapath's arithmetic: no reduction, no
layout offsets, no partitioning. Element conversion to bf16/fp16 is done by
numpy/torch (plumbing), never by the library or the oracle.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-style. A stream is keyed by
(seed, cfg, buf); its key is the first SplitMix64 output from the state
``seed ^ (cfg << 32) ^ buf``, and value k of the stream is the SplitMix64
finaliser applied to ``key + (k + 1) * GAMMA``: exactly the (k+1)-th output
of a SplitMix64 generator seeded with ``key``. Every value depends only on
(seed, cfg, buf, k), so any slice of a stream can be generated on its own, on
the host (numpy) or on a device (torch), with identical bits.

Distributions (values per element k of a buffer):
- ``uniform_pm1``: u = (r >> 40) * 2^-24, x = 2u - 1 (exact in fp32), then
  round-to-nearest-even into the element type.
- ``normal``: Box-Muller in float64 from r_{2k}, r_{2k+1}:
  u1 = ((r_{2k} >> 11) + 1) * 2^-53 in (0, 1], u2 = (r_{2k+1} >> 11) * 2^-53,
  z = sqrt(-2 ln u1) * cos(2 pi u2); x = sigma * z -> fp32 -> element type.
  libm differences between hosts/devices may flip a last bit; both sides of a
  parity check always consume the same stored bytes, so this never matters.
- ``bits``: raw 64-bit outputs laid out little-endian as bytes.
- ``categorical``: u = (r >> 11) * 2^-53, category = first d with u < CDF[d],
  the last CDF entry forced to 1.
"""
from __future__ import annotations

import math

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1


def zipf_weights(s: float, n: int) -> np.ndarray:
    """Weights proportional to (d+1)^-s for d = 0..n-1, normalised (float64)."""
    w = np.array([(d + 1) ** (-s) for d in range(n)], dtype=np.float64)
    return w / w.sum()


def zipf_split(total: int, n: int = 8, s: float = 0.125, granule: int = 16) -> list:
    """Partition sizes (bytes) of a variable-length collective of total message size
    `total` over n ranks (Purlin paper, appendix C.4: rank r gets a Zipf-split share
    with exponent s = 0.125; splits preserve the total; 1 and 2 KiB totals are split
    uniformly). Reading: below 4 KiB every rank gets total / n; otherwise rank r's
    weight is (r+1)^-s normalised, every share is rounded down to a multiple of
    `granule` bytes (the datapath's 16-byte alignment), and the granules left over go
    one each to ranks 0, 1, 2, ... so that shares never increase with r. `total` must
    be a multiple of n * granule."""
    if total % (n * granule):
        raise ValueError("total must be a multiple of n * granule")
    if total < 4096:
        return [total // n] * n
    w = zipf_weights(s, n)
    parts = [int(total * float(w[r])) // granule * granule for r in range(n)]
    left = (total - sum(parts)) // granule
    for r in range(left):
        parts[r % n] += granule
    return parts


# --------------------------------------------------------------------------
# Scalar reference of the generator (pure Python ints), used to pin both
# vectorised backends.
# --------------------------------------------------------------------------
def _mix_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, cfg: int, buf: int) -> int:
    state = (seed ^ (cfg << 32) ^ buf) & MASK64
    return _mix_int(state + GAMMA)


def stream_value_int(seed: int, cfg: int, buf: int, k: int) -> int:
    """Value k of stream (seed, cfg, buf), as a Python int."""
    return _mix_int(stream_key(seed, cfg, buf) + (k + 1) * GAMMA)


# --------------------------------------------------------------------------
# numpy backend (host)
# --------------------------------------------------------------------------
def _mix_np(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
    return z ^ (z >> np.uint64(31))


def raw_np(seed: int, cfg: int, buf: int, count: int, start: int = 0) -> np.ndarray:
    """uint64 values start .. start+count-1 of the stream."""
    key = np.uint64(stream_key(seed, cfg, buf))
    k = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix_np(key + k * np.uint64(GAMMA))


def _to_dtype_np(x32: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values -> raw element bits (uint16 for bf16/f16, float32 for f32)."""
    if dtype == "f32":
        return x32.astype(np.float32)
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def uniform_pm1_np(seed, cfg, buf, n, dtype="bf16", start=0):
    r = raw_np(seed, cfg, buf, n, start)
    u = (r >> np.uint64(40)).astype(np.float64) * 2.0**-24
    return _to_dtype_np((2.0 * u - 1.0).astype(np.float32), dtype)


def normal_np(seed, cfg, buf, n, sigma=1.0, dtype="bf16", start=0):
    r = raw_np(seed, cfg, buf, 2 * n, 2 * start)
    u1 = ((r[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0**-53
    u2 = (r[1::2] >> np.uint64(11)).astype(np.float64) * 2.0**-53
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)
    return _to_dtype_np((sigma * z).astype(np.float32), dtype)


def bits_np(seed, cfg, buf, nbytes, start_byte=0):
    """nbytes random bytes (nbytes and start_byte multiples of 8)."""
    assert nbytes % 8 == 0 and start_byte % 8 == 0
    return raw_np(seed, cfg, buf, nbytes // 8, start_byte // 8).view(np.uint8)


def categorical_np(seed, cfg, buf, n, probs, start=0):
    cdf = np.cumsum(np.asarray(probs, dtype=np.float64))
    cdf[-1] = 1.0
    r = raw_np(seed, cfg, buf, n, start)
    u = (r >> np.uint64(11)).astype(np.float64) * 2.0**-53
    return np.searchsorted(cdf, u, side="right").astype(np.int32)


# --------------------------------------------------------------------------
# torch backend (any device; int64 with two's-complement wrap-around)
# --------------------------------------------------------------------------
def _s64(x: int) -> int:
    x &= MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


def _lsr(t, k: int):
    import torch

    return torch.bitwise_and(t >> k, (1 << (64 - k)) - 1)


def _mix_t(z):
    z = (z ^ _lsr(z, 30)) * _s64(M1)
    z = (z ^ _lsr(z, 27)) * _s64(M2)
    return z ^ _lsr(z, 31)


def raw_t(seed, cfg, buf, count, start=0, device="cpu"):
    """int64 tensor holding the bits of values start .. start+count-1."""
    import torch

    key = _s64(stream_key(seed, cfg, buf))
    k = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    return _mix_t(k * _s64(GAMMA) + key)


def _top_bits_t(r, drop: int):
    """(r >> drop) as a non-negative int64, as float64."""
    return _lsr(r, drop).to(__import__("torch").float64)


def _to_dtype_t(x32, dtype):
    import torch

    if dtype == "f32":
        return x32
    if dtype == "f16":
        return x32.to(torch.float16)
    if dtype == "bf16":
        return x32.to(torch.bfloat16)
    raise ValueError(dtype)


def uniform_pm1_t(seed, cfg, buf, n, dtype="bf16", start=0, device="cpu"):
    import torch

    u = _top_bits_t(raw_t(seed, cfg, buf, n, start, device), 40) * 2.0**-24
    return _to_dtype_t((2.0 * u - 1.0).to(torch.float32), dtype)


def normal_t(seed, cfg, buf, n, sigma=1.0, dtype="bf16", start=0, device="cpu"):
    import torch

    r = raw_t(seed, cfg, buf, 2 * n, 2 * start, device)
    u1 = (_top_bits_t(r[0::2], 11) + 1.0) * 2.0**-53
    u2 = _top_bits_t(r[1::2], 11) * 2.0**-53
    z = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * math.pi * u2)
    return _to_dtype_t((sigma * z).to(torch.float32), dtype)


def bits_t(seed, cfg, buf, nbytes, start_byte=0, device="cpu"):
    """uint8 tensor of nbytes random bytes (same bytes as bits_np)."""
    import torch

    assert nbytes % 8 == 0 and start_byte % 8 == 0
    return raw_t(seed, cfg, buf, nbytes // 8, start_byte // 8, device).view(torch.uint8)


def categorical_t(seed, cfg, buf, n, probs, start=0, device="cpu"):
    import torch

    cdf = np.cumsum(np.asarray(probs, dtype=np.float64))
    cdf[-1] = 1.0
    u = _top_bits_t(raw_t(seed, cfg, buf, n, start, device), 11) * 2.0**-53
    c = torch.tensor(cdf, dtype=torch.float64, device=device)
    return torch.searchsorted(c, u, right=True).to(torch.int32)
