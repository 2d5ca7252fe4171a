"""Helpers shared by the GPU tests: moving raw element bits between numpy and device
tensors, and NaN-as-a-class comparison. No datapath arithmetic lives here."""
import numpy as np
import torch

NP_RAW = {"bf16": np.uint16, "f16": np.uint16, "f32": np.uint32}


def to_dev(a: np.ndarray) -> torch.Tensor:
    """Raw bytes of a numpy array -> a uint8 device tensor (16-byte aligned allocation)."""
    b = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
    return torch.from_numpy(b.copy()).cuda()


def from_dev(t: torch.Tensor, dtype=np.uint8) -> np.ndarray:
    return t.cpu().numpy().reshape(-1).view(np.uint8).view(dtype)


def empty_dev(nbytes: int, fill: int | None = None) -> torch.Tensor:
    t = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    if fill is not None:
        t.fill_(fill)
    return t


def nan_mask(dtype, p):
    if dtype == "bf16":
        return ((p & 0x7F80) == 0x7F80) & ((p & 0x7F) != 0)
    if dtype == "f16":
        return ((p & 0x7C00) == 0x7C00) & ((p & 0x3FF) != 0)
    return ((p & 0x7F800000) == 0x7F800000) & ((p & 0x7FFFFF) != 0)


def assert_same(dtype, got, ref, what=""):
    """Bitwise equality with NaN compared as a class (any NaN matches any NaN)."""
    raw = NP_RAW[dtype]
    g = np.ascontiguousarray(got).reshape(-1).view(raw)
    r = np.ascontiguousarray(ref).reshape(-1).view(raw)
    assert g.size == r.size, (what, g.size, r.size)
    gn, rn = nan_mask(dtype, g), nan_mask(dtype, r)
    bad = (gn != rn) | (~gn & (g != r))
    if bad.any():
        i = np.flatnonzero(bad)
        raise AssertionError(f"{what}: {i.size} mismatches, first at {i[:5]}: "
                             f"got {[hex(int(x)) for x in g[i[:5]]]} want {[hex(int(x)) for x in r[i[:5]]]}")
