"""The fused AdamW step's entry point that allocates no device memory,
fsdp_adamw_shard_step_noalloc, against the allocating fsdp_adamw_shard_step
on the same inputs (through the C ABI): bit for bit, on two calls in a row,
the second on a smaller unit, then the first unit again (its table goes back
into the shared static buffer); and the refusal of a table beyond that
buffer, before any device work."""

import ctypes

import numpy as np
import pytest
import torch

import fully_sharded_amd as F
from tests.gpu_util import assert_bitexact, to_dev, to_host
from workloads.configs import ADAMW, BLOCK_512, shapes_of

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    F.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def banner(msg):
    print(f"[gpu] {msg}", flush=True)


def unit_inputs(plan, seed):
    """Seeded state (master, m, v with m, v non-zero) and R bf16 gradient
    replicas for one unit; the padding of the state is +0."""
    rng = np.random.default_rng(seed)
    n = plan.R * plan.S
    master = rng.uniform(-0.05, 0.05, n).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.uniform(0.0, 1e-7, n)).astype(np.float32)
    grads = []
    for _ in range(plan.R):
        g = (rng.standard_normal(plan.T) * 1e-3).astype(np.float32)
        grads.append((g.view(np.uint32) >> 16).astype(np.uint16))   # bf16 by truncation
    return master, m, v, grads


def both_entry_points(plan, inputs, step):
    """One step through each entry point from identical device copies."""
    master, m, v, grads = inputs
    g = [to_dev(x) for x in grads]
    outs = []
    for fn in (F.fsdp_adamw_shard_step, F.fsdp_adamw_shard_step_noalloc):
        st = [to_dev(master), to_dev(m), to_dev(v)]
        param = torch.empty(plan.R * plan.S, dtype=torch.bfloat16, device=DEV)
        fn(plan, ADAMW, step, g, st[0], st[1], st[2], param)
        torch.cuda.synchronize()
        outs.append([to_host(t) for t in st] + [to_host(param)])
    return outs


def test_noalloc_matches_the_allocating_step_on_consecutive_calls():
    # two blocks at R = 8: 6,146 work items, the capped two-element launch;
    # one block: 3,130, the one-element launch; ragged R = 3: two-element
    two = F.Plan(shapes_of(BLOCK_512) * 2, 8, "per_param")
    big = F.Plan(shapes_of(BLOCK_512), 8, "per_param")
    small = F.Plan([(300, 17), (45,), (1000, 3)], 3, "per_param")
    assert len(small.work_items(0)) < len(big.work_items(0)) < 4096 < len(two.work_items(0))
    for what, plan, seed, step in (("two blocks R=8", two, 6, 2), ("block R=8 (smaller)", big, 1, 3),
                                   ("ragged R=3 (smaller)", small, 2, 2),
                                   ("block R=8 again", big, 3, 5)):
        banner(f"noalloc vs allocating step: {what}")
        ref, got = both_entry_points(plan, unit_inputs(plan, seed), step)
        for name, a, b in zip(("master", "m", "v", "param"), got, ref):
            assert_bitexact(a, b, f"{what} {name}")


def test_noalloc_unfused_step_matches():
    banner("noalloc vs allocating step, reduced fp32 gradient")
    plan = F.Plan(shapes_of(BLOCK_512), 4, "per_param")
    master, m, v, _ = unit_inputs(plan, 4)
    rng = np.random.default_rng(5)
    red = to_dev((rng.standard_normal(plan.R * plan.S) * 1e-3).astype(np.float32))
    outs = []
    for fn in (F.fsdp_adamw_shard_step, F.fsdp_adamw_shard_step_noalloc):
        st = [to_dev(master), to_dev(m), to_dev(v)]
        param = torch.empty(plan.R * plan.S, dtype=torch.bfloat16, device=DEV)
        fn(plan, ADAMW, 2, [red], st[0], st[1], st[2], param, grads_are_replicas=False)
        torch.cuda.synchronize()
        outs.append([to_host(t) for t in st] + [to_host(param)])
    for name, a, b in zip(("master", "m", "v", "param"), outs[1], outs[0]):
        assert_bitexact(a, b, f"unfused {name}")


def test_noalloc_refuses_a_table_beyond_its_buffer():
    banner("noalloc refuses a plan with more than 43,690 work items")
    plan = F.Plan([(50_000_000,)], 1, "flat")              # 48,829 work items
    assert len(plan.work_items(0)) > 43690
    h = F.binding.AdamWHParams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    arr = (ctypes.c_void_p * 1)(None)
    # refused before any argument is looked at or any device call is made
    rc = F.lib().fsdp_adamw_shard_step_noalloc(plan.handle, ctypes.byref(h), 1, arr, 1, 1,
                                               None, None, None, None, 1, None)
    assert rc == -2
