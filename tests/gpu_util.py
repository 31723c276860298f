"""Helpers shared by the GPU tests: host <-> device transfers of bf16 bit
patterns, and the comparison bars (bit-exact, AdamW tolerance, bf16 ulp)."""

import numpy as np
import torch


def to_dev(a: np.ndarray, device="cuda"):
    """Host array (fp32, or uint16 bf16 bits) -> device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array (bf16 as uint16 bits)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def assert_bitexact(got: np.ndarray, want: np.ndarray, what=""):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    g, w = bits(got), bits(want)
    if not np.array_equal(g, w):
        bad = np.flatnonzero(g.reshape(-1) != w.reshape(-1))
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {g.size} differ; first at {i}: "
                             f"got {hex(int(g.reshape(-1)[i]))} want {hex(int(w.reshape(-1)[i]))}")


def assert_adamw_close(got: np.ndarray, want: np.ndarray, what=""):
    """max |got - want| <= 1e-6 * max(1, |want|), NaN only where NaN."""
    g = got.astype(np.float64)
    w = want.astype(np.float64)
    gn, wn = np.isnan(g), np.isnan(w)
    assert np.array_equal(gn, wn), f"{what}: NaN pattern differs"
    ok = ~wn
    tol = 1e-6 * np.maximum(1.0, np.abs(w[ok]))
    d = np.abs(g[ok] - w[ok])
    same_inf = np.isinf(w[ok]) & (g[ok] == w[ok])
    bad = (d > tol) & ~same_inf
    assert not bad.any(), f"{what}: {bad.sum()} beyond tolerance, worst {d.max():.3e}"


def bf16_order(u: np.ndarray) -> np.ndarray:
    u = u.astype(np.int64)
    return np.where(u & 0x8000, -(u & 0x7FFF), u)


def assert_bf16_within_ulp(got: np.ndarray, want: np.ndarray, what=""):
    """bf16 bit patterns within one ulp of each other (NaN only where NaN)."""
    gn = (got & 0x7FFF) > 0x7F80
    wn = (want & 0x7FFF) > 0x7F80
    assert np.array_equal(gn, wn), f"{what}: NaN pattern differs"
    d = np.abs(bf16_order(got[~gn]) - bf16_order(want[~wn]))
    assert d.max(initial=0) <= 1, f"{what}: bf16 differs by {d.max()} ulp"
