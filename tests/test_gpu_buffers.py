"""The placement helpers with the library: arrays carved by
fully_sharded_amd.unit_buffers / rows (rows of one buffer, strides off
multiples of 4 KiB) pass the library's overlap checks and give, bit for bit,
the results of the same calls on one allocation per array, for a ragged
per-parameter unit at R = 3 and the 12-layer model's block at R = 8."""

import numpy as np
import pytest
import torch

import fully_sharded_amd as F
from tests.gpu_util import assert_bitexact, to_dev, to_host
from workloads.configs import ADAMW

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("shapes,R,layout", [
    ([(67, 5), (130,), (9, 4, 3)], 3, "per_param"),
    ([(512, 512)] * 4 + [(512, 2048), (2048, 512), (512,), (512,)], 8, "per_param"),
])
def test_carved_buffers_match_separate_allocations(shapes, R, layout):
    print(f"[gpu] buffers R={R} {layout}", flush=True)
    rng = np.random.default_rng(900 + R)
    plan = F.Plan(shapes, R, layout)
    n = plan.R * plan.S
    full = to_dev(rng.uniform(-0.5, 0.5, plan.T).astype(np.float32))
    grads_h = [(rng.standard_normal(plan.T) * 1e-3).astype(np.float32) for _ in range(R)]

    carved = F.unit_buffers(plan, torch.bfloat16, torch.bfloat16, DEV)
    separate = (torch.empty(n, device=DEV), torch.empty(n, device=DEV),
                torch.empty(n, device=DEV), torch.empty(n, dtype=torch.bfloat16, device=DEV),
                [torch.empty(plan.T, dtype=torch.bfloat16, device=DEV) for _ in range(R)])
    recvs = []
    for master, m, v, param, grads in (carved, separate):
        m.zero_()
        v.zero_()
        F.fsdp_shard_pack(plan, full, master)
        F.fsdp_shard_pack(plan, full, param)
        for g, h in zip(grads, grads_h):
            g.copy_(to_dev(h).bfloat16())
        recv = F.rows(R, plan.T, torch.bfloat16, DEV)
        for t in (1, 2):
            F.fsdp_gather_unflatten(plan, param, recv)
            F.fsdp_adamw_shard_step(plan, ADAMW, t, grads, master, m, v, param)
        recvs.append(recv)
    torch.cuda.synchronize()
    for name, a, b in zip(("master", "m", "v", "param"), carved[:4], separate[:4]):
        assert_bitexact(to_host(a), to_host(b), name)
    assert np.any(to_host(carved[1]) != 0)
    for r in range(R):
        assert_bitexact(to_host(recvs[0][r]), to_host(recvs[1][r]), f"receiver {r}")
