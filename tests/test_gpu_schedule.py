"""The unit loop's schedules give the same state bit for bit: the prefetch
schedule (gathers on their own stream, double receive buffer) and two
gathers per step change ordering and traffic, not results."""

import pytest
import torch

import fully_sharded_amd as F
from fully_sharded_amd.step import StepRunner, Unit
from workloads import gen
from workloads.configs import ADAMW, WORKLOADS, shapes_of

pytestmark = pytest.mark.gpu
DEV = "cuda"


def build(wl_name, n_units=None):
    wl = WORKLOADS[wl_name]
    R = wl["R"]
    shapes = shapes_of(wl["units"][0])
    pl = F.Plan(shapes, R, wl["layout"])
    units = []
    for u in range(n_units or len(wl["units"])):
        full = gen.device_master(wl, u, shapes, DEV)
        master = torch.empty(R * pl.S, device=DEV)
        F.fsdp_shard_pack(pl, full, master)
        param = torch.empty(R * pl.S, dtype=torch.bfloat16, device=DEV)
        F.fsdp_shard_pack(pl, full, param)
        grads = [gen.device_grad(wl, 1, u, r, pl.T, DEV) for r in range(R)]
        units.append(Unit(pl, master, torch.zeros_like(master), torch.zeros_like(master),
                          param, grads))
    recv = [[torch.empty(pl.T, dtype=torch.bfloat16, device=DEV) for _ in range(R)]
            for _ in range(2)]
    return units, recv


def state_of(units):
    return [(u.master.clone(), u.m.clone(), u.v.clone(), u.param.view(torch.int16).clone())
            for u in units]


@pytest.mark.parametrize("schedule,gathers", [("prefetch", 1), ("serial", 2), ("prefetch", 2)])
def test_schedules_agree_bit_for_bit(schedule, gathers):
    print(f"[gpu] schedule={schedule} gathers={gathers}", flush=True)
    ref_units, ref_recv = build("model12_r8")
    ref = StepRunner(ref_units, ADAMW, ref_recv, "serial", 1)
    units, recv = build("model12_r8")
    run = StepRunner(units, ADAMW, recv, schedule, gathers)
    for t in (1, 2, 3):
        ref.step(t)
        run.step(t)
    torch.cuda.synchronize()
    for a, b in zip(state_of(ref_units), state_of(units)):
        for x, y in zip(a, b):
            assert torch.equal(x, y)
    # the receive buffers hold the last gathered units, the same in both runs
    n = len(units)
    last = recv[(n - 1) % 2] if schedule == "prefetch" else recv[0]
    for r in range(len(last)):
        assert torch.equal(last[r].view(torch.int16), ref_recv[0][r].view(torch.int16))


def test_memory_ledger_counts_the_prefetch_buffer():
    units, recv = build("model12_r8", n_units=3)
    serial = StepRunner(units, ADAMW, recv, "serial").memory_ledger()
    pre = StepRunner(units, ADAMW, recv, "prefetch").memory_ledger()
    T, S = units[0].plan.T, units[0].plan.S
    assert serial["sharded_state"] == 3 * 16 * S
    assert serial["largest_unsharded_group"] == 2 * T and serial["prefetch"] == 0
    assert pre["prefetch"] == 2 * T
    assert pre["peak_lower_bound"] == serial["peak_lower_bound"] + 2 * T
