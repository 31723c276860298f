"""Randomised sequences through the C ABI against the oracle: random small
units (1-4 parameters, 1-3 dims, dims 1-70), random R (1-16) and layouts;
per case pack, two steps through the paired step-then-gather call and a
third through the standalone fused step, a re-shard of the trained state to
another R and layout, the averaged all-reduce and a two-micro-batch
accumulation.  Bit-exact wherever the contract says so, AdamW to its
tolerance and, since the kernels evaluate it as the oracle does, bit for
bit.

The environment can widen the run: FSDP_RANDOM_SEEDS (number of sequences,
24 by default), FSDP_RANDOM_RMAX (largest R, 16) and FSDP_RANDOM_DMAX
(largest leading dimension, 70), e.g.
FSDP_RANDOM_SEEDS=1000 python -m pytest -m gpu tests/test_gpu_random.py."""

import os

import numpy as np
import pytest
import torch

import fully_sharded_amd as F
from oracle import fsdp_oracle as O
from tests.gpu_util import (assert_adamw_close, assert_bf16_within_ulp, assert_bitexact,
                            to_dev, to_host)
from workloads.configs import ADAMW

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    F.lib()
    yield
    torch.cuda.synchronize()


N_SEEDS = int(os.environ.get("FSDP_RANDOM_SEEDS", "24"))
R_MAX = int(os.environ.get("FSDP_RANDOM_RMAX", "16"))
D_MAX = int(os.environ.get("FSDP_RANDOM_DMAX", "70"))


def random_shapes(rng):
    """1-4 parameters; the leading dimension up to D_MAX, the others up to 70
    (at most two dimensions when D_MAX > 70, to bound the size)."""
    out = []
    for _ in range(int(rng.integers(1, 5))):
        nd = int(rng.integers(1, 4 if D_MAX <= 70 else 3))
        out.append((int(rng.integers(1, D_MAX + 1)),) +
                   tuple(int(x) for x in rng.integers(1, 71, nd - 1)))
    return out


def random_unit(rng, R, layout):
    shapes = random_shapes(rng)
    po = O.plan_layout(shapes, R, layout)
    full = rng.uniform(-1, 1, po.T).astype(np.float32)
    grads = [O.bf16_rne((rng.standard_normal(po.T) * 1e-2).astype(np.float32))
             for _ in range(R)]
    return shapes, po, full, grads


@pytest.mark.parametrize("seed", list(range(N_SEEDS)))
def test_random_sequence_matches_the_oracle(seed):
    rng = np.random.default_rng(9000 + seed)
    R = int(rng.integers(1, R_MAX + 1))
    layout = ["per_param", "flat"][int(rng.integers(0, 2))]
    print(f"[gpu] random seed={seed} R={R} {layout}", flush=True)
    shapes, po, full, grads = random_unit(rng, R, layout)
    nshapes, npo, nfull, _ = random_unit(rng, R, ["per_param", "flat"][int(rng.integers(0, 2))])
    pg, npg = F.Plan(shapes, R, layout), F.Plan(nshapes, R, npo.layout)

    # pack: fp32 master exactly, bf16 parameter through RNE
    master = torch.empty(R * po.S, device=DEV)
    param = torch.empty(R * po.S, dtype=torch.bfloat16, device=DEV)
    F.fsdp_shard_pack(pg, to_dev(full), master)
    F.fsdp_shard_pack(pg, to_dev(full), param)
    mo = O.shard_pack(po, full)
    assert_bitexact(to_host(master).reshape(R, po.S), mo, "pack f32")
    assert_bitexact(to_host(param).reshape(R, po.S), O.bf16_rne(mo), "pack bf16")
    nparam = torch.empty(R * npo.S, dtype=torch.bfloat16, device=DEV)
    F.fsdp_shard_pack(npg, to_dev(nfull), nparam)
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    recv = [torch.empty(npo.T, dtype=torch.bfloat16, device=DEV) for _ in range(R)]
    g_d = [to_dev(g) for g in grads]

    # two steps, each with the next unit's gather in the same call
    om, ov = np.zeros_like(mo), np.zeros_like(mo)
    for t in (1, 2):
        F.fsdp_adamw_step_then_gather(pg, ADAMW, t, g_d, master, m, v, param, npg, nparam, recv)
        mo, om, ov, po_param = O.shard_step(po, grads, mo, om, ov, t, ADAMW, "bf16")
        torch.cuda.synchronize()
        gm = to_host(master).reshape(R, po.S)
        assert_adamw_close(gm, mo, f"master t={t}")
        assert_adamw_close(to_host(m).reshape(R, po.S), om, f"m t={t}")
        assert_adamw_close(to_host(v).reshape(R, po.S), ov, f"v t={t}")
        gp = to_host(param).reshape(R, po.S)
        assert_bf16_within_ulp(gp, po_param, f"param t={t}")
        assert_bitexact(gp, O.bf16_rne(gm), "param = RNE(master)")
        assert_bitexact(gm, mo, f"master bits t={t}")
        assert_bitexact(gp, po_param, f"param bits t={t}")
        want, _ = O.gather_unflatten(npo, O.bf16_rne(O.shard_pack(npo, nfull)))
        for r in recv:
            assert_bitexact(to_host(r), want, "next unit's gather")

    # a third step through the standalone fused call (at this size the
    # two-element kernel at R = 3 or 4, the one-element kernel at R >= 8)
    F.fsdp_adamw_shard_step(pg, ADAMW, 3, g_d, master, m, v, param)
    mo, om, ov, po_param = O.shard_step(po, grads, mo, om, ov, 3, ADAMW, "bf16")
    torch.cuda.synchronize()
    assert_bitexact(to_host(master).reshape(R, po.S), mo, "master t=3")
    assert_bitexact(to_host(m).reshape(R, po.S), om, "m t=3")
    assert_bitexact(to_host(v).reshape(R, po.S), ov, "v t=3")
    assert_bitexact(to_host(param).reshape(R, po.S), po_param, "param t=3")

    # re-shard the trained fp32 state to another world size and layout
    R2 = int(rng.integers(1, R_MAX + 1))
    l2 = ["per_param", "flat"][int(rng.integers(0, 2))]
    po2 = O.plan_layout(shapes, R2, l2)
    rs = F.Resharder(pg, F.Plan(shapes, R2, l2))
    outs = [torch.full((R2 * po2.S,), 9.0, device=DEV) for _ in range(3)]
    F.fsdp_reshard_batch(rs, [master, m, v], outs)
    for got, src in zip(outs, (master, m, v)):
        assert_bitexact(to_host(got).reshape(R2, po2.S),
                        O.reshard(po, po2, to_host(src).reshape(R, po.S)), "reshard")

    # DDP's averaged all-reduce and a two-micro-batch accumulation
    ar = [torch.empty(po.T, device=DEV) for _ in range(R)]
    F.fsdp_allreduce_avg(pg, g_d, ar)
    want = O.allreduce_avg(grads)
    for a, w in zip(ar, want):
        assert_bitexact(to_host(a), w, "all-reduce")
    acc = [torch.empty(po.T, device=DEV) for _ in range(R)]
    F.fsdp_grad_accumulate(pg, g_d, acc, True)
    F.fsdp_grad_accumulate(pg, g_d[::-1], acc, False)
    for r in range(R):
        assert_bitexact(to_host(acc[r]), O.grad_accumulate([grads[r], grads[R - 1 - r]]),
                        "accumulate")
