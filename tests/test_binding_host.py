"""Host-side checks of the Python binding (no GPU): it refuses host tensors,
wrong sizes and dtypes before calling the library, and nothing in it
computes a result on the CPU."""

import pytest
import torch

import fully_sharded_amd as F
from workloads.configs import ADAMW


@pytest.fixture
def plan():
    return F.Plan([(6, 4), (5,)], 2, "per_param")


def test_host_tensors_are_refused(plan):
    shards = torch.zeros(plan.R * plan.S, dtype=torch.bfloat16)
    recv = [torch.zeros(plan.T, dtype=torch.bfloat16) for _ in range(plan.R)]
    with pytest.raises(ValueError, match="GPU tensor"):
        F.fsdp_gather_unflatten(plan, shards, recv)
    full = torch.zeros(plan.T)
    with pytest.raises(ValueError, match="GPU tensor"):
        F.fsdp_shard_pack(plan, full, torch.zeros(plan.R * plan.S))


def test_sizes_and_dtypes_are_checked_first(plan):
    n = plan.R * plan.S
    st = [torch.zeros(n) for _ in range(3)]
    grads = [torch.zeros(plan.T, dtype=torch.bfloat16) for _ in range(plan.R)]
    with pytest.raises(ValueError):          # one gradient too few
        F.bind_adamw_shard_step(plan, ADAMW, grads[:1], *st, torch.zeros(n, dtype=torch.bfloat16))
    with pytest.raises(ValueError):          # master not fp32
        F.bind_adamw_shard_step(plan, ADAMW, grads, st[0].bfloat16(), st[1], st[2],
                                torch.zeros(n, dtype=torch.bfloat16))
    with pytest.raises(ValueError):          # the reduced gradient must be fp32 [R*S]
        F.bind_adamw_shard_step(plan, ADAMW, torch.zeros(n - 1), *st,
                                torch.zeros(n, dtype=torch.bfloat16), grads_are_replicas=False)
    with pytest.raises(ValueError):          # receiver too short
        F.bind_gather_unflatten(plan, torch.zeros(n, dtype=torch.bfloat16),
                                [torch.zeros(plan.T - 1, dtype=torch.bfloat16)] * plan.R)
    with pytest.raises(ValueError):          # next unit's shards in another dtype
        F.bind_adamw_step_then_gather(plan, ADAMW, grads, *st, torch.zeros(n, dtype=torch.bfloat16),
                                      plan, torch.zeros(n), [torch.zeros(plan.T)] * plan.R)
    with pytest.raises(TypeError):           # fp16 is not a dtype of the ABI
        F.fsdp_reduce_scatter_avg(plan, [g.half() for g in grads], torch.zeros(n))
    with pytest.raises(ValueError):
        F.fsdp_reshard_batch(F.Resharder(plan, F.Plan([(6, 4), (5,)], 3, "flat")), [], [])


def test_plan_views_without_a_gpu(plan):
    full = torch.arange(plan.T, dtype=torch.float32)
    w, b = plan.unflatten(full)
    assert w.shape == (6, 4) and b.shape == (5,)
    assert w.data_ptr() == full.data_ptr()            # views, no copy
    assert torch.equal(b, torch.arange(24, 29, dtype=torch.float32))


def test_unit_buffers_carve_rows_off_4k_strides(plan):
    master, m, v, param, grads = F.unit_buffers(plan, torch.bfloat16, torch.bfloat16, "cpu")
    n = plan.R * plan.S
    assert [t.numel() for t in (master, m, v, param)] == [n] * 4
    assert master.dtype == m.dtype == v.dtype == torch.float32 and param.dtype == torch.bfloat16
    assert len(grads) == plan.R and all(g.numel() == plan.T for g in grads)
    assert all(g.dtype == torch.bfloat16 for g in grads)
    for row in ([master, m, v], grads):
        bases = [t.data_ptr() for t in row]
        steps = {b - a for a, b in zip(bases, bases[1:])}
        assert len(steps) == 1
        step = steps.pop()
        assert step % 256 == 0 and step % 4096 != 0 and step >= row[0].numel() * row[0].element_size()
    # rows of one buffer: 4 KiB rows get 256 B more, short rows round to 256 B
    a = F.rows(3, 1024, torch.float32, "cpu")
    assert a[1].data_ptr() - a[0].data_ptr() == 4096 + 256
    c = F.rows(2, 100, torch.bfloat16, "cpu")
    assert c[1].data_ptr() - c[0].data_ptr() == 256
