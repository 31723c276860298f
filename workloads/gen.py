"""Seeded synthetic inputs for the FSDP workloads.

Every input -- per-rank gradients and initial fp32 master weights -- comes
from here, keyed by (workload id, step, unit, rank, kind), so the oracle and
the GPU path always see identical bits.  Nothing in this module computes any
part of the method: values are drawn, scaled to the stated distribution and
stored in the requested dtype (bf16 through torch's own float->bfloat16 cast).

Two sources with the same keys:
  * host: numpy ``default_rng`` seeded per fixed 1 Mi-element chunk, so any
    sub-range can be regenerated on its own;
  * device: a torch generator on the GPU, for workloads too large to draw on
    the host in reasonable time.  Its values differ from the host source; a
    test reads device-drawn inputs back to the host when the oracle needs them.

Distributions (the pages print none; these are the stated readings):
  * gradients: N(0, sigma) with sigma from the workload (1.0 for the toy,
    1e-3 for the transformer workloads);
  * masters: U(-1/sqrt(fan_in), +1/sqrt(fan_in)) with fan_in = shape[1] for a
    2-D weight, 1.0 for a 1-D LayerNorm scale, N(0, 1) for the toy;
  * Adam moments start at zero.
"""

from __future__ import annotations

import math

import numpy as np

CHUNK = 1 << 20
KIND_GRAD = 0
KIND_MASTER = 1


def _seed_int(key) -> int:
    ss = np.random.SeedSequence([0] + [int(k) for k in key])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64((1 << 63) - 1))


def host_normal(key, n: int, sigma: float) -> np.ndarray:
    """N(0, sigma) fp32 values, drawn chunk by chunk."""
    out = np.empty(n, np.float32)
    for c in range((n + CHUNK - 1) // CHUNK):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        rng = np.random.default_rng([0] + [int(k) for k in key] + [c])
        out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)
    if sigma != 1.0:
        out *= np.float32(sigma)
    return out


def host_uniform(key, n: int, bound: float) -> np.ndarray:
    """U(-bound, bound) fp32 values, drawn chunk by chunk."""
    out = np.empty(n, np.float32)
    for c in range((n + CHUNK - 1) // CHUNK):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        rng = np.random.default_rng([0] + [int(k) for k in key] + [c])
        out[lo:hi] = rng.uniform(-bound, bound, hi - lo).astype(np.float32)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32 values, via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def host_grad(wl: dict, step: int, unit: int, rank: int, n: int) -> np.ndarray:
    """One rank's full-unit gradient: fp32, or bf16 bits (uint16)."""
    g = host_normal((wl["cid"], step, unit, rank, KIND_GRAD), n, wl["grad_sigma"])
    return to_bf16_bits(g) if wl["grad_dtype"] == "bf16" else g


def host_master(wl: dict, unit: int, shapes) -> np.ndarray:
    """Initial fp32 master of one unit, as its full-unit (flattened) buffer."""
    parts = []
    for p, shape in enumerate(shapes):
        n = 1
        for d in shape:
            n *= int(d)
        key = (wl["cid"], 0, unit, p, KIND_MASTER)
        if wl["master_init"] == "normal":
            parts.append(host_normal(key, n, 1.0))
        elif len(shape) == 1:
            parts.append(np.ones(n, np.float32))
        else:
            parts.append(host_uniform(key, n, 1.0 / math.sqrt(shape[1])))
    return np.concatenate(parts) if parts else np.zeros(0, np.float32)


# ---------------------------------------------------------------- device side
def device_normal(key, n: int, sigma: float, device, dtype):
    """N(0, sigma) drawn on the GPU by torch, stored as ``dtype``."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_seed_int(key))
    x = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(dtype)


def device_grad(wl: dict, step: int, unit: int, rank: int, n: int, device):
    import torch
    dt = torch.bfloat16 if wl["grad_dtype"] == "bf16" else torch.float32
    return device_normal((wl["cid"], step, unit, rank, KIND_GRAD), n,
                         wl["grad_sigma"], device, dt)


def device_master(wl: dict, unit: int, shapes, device):
    """Initial fp32 master of one unit drawn on the GPU (full-unit buffer)."""
    import torch
    parts = []
    for p, shape in enumerate(shapes):
        n = 1
        for d in shape:
            n *= int(d)
        if wl["master_init"] == "normal":
            parts.append(device_normal((wl["cid"], 0, unit, p, KIND_MASTER), n,
                                       1.0, device, torch.float32))
        elif len(shape) == 1:
            parts.append(torch.ones(n, device=device, dtype=torch.float32))
        else:
            g = torch.Generator(device=device)
            g.manual_seed(_seed_int((wl["cid"], 0, unit, p, KIND_MASTER)))
            b = 1.0 / math.sqrt(shape[1])
            x = torch.rand(n, generator=g, device=device, dtype=torch.float32)
            parts.append(x.mul_(2 * b).sub_(b))
    return torch.cat(parts)
