"""The stream entry points under HIP stream capture.

A caller may record the library's calls into its own graph (torch's
CUDAGraph here) once the plans' work tables are on the device
(fsdp_plan_prepare): every call is kernel launches only, with no
allocation, copy or memset on the stream.  A short unit loop -- gather of
unit 0, unit 0's step together with unit 1's gather, unit 1's step, a
reduce-scatter and a re-shard -- is captured once and replayed several
times, with eager work and synchronisations between the replays; after
every replay each buffer equals, bit for bit, the same calls run eagerly the
same number of times on a copy of the inputs."""

import numpy as np
import pytest
import torch

import fully_sharded_amd as F
from tests.gpu_util import assert_bitexact, to_dev, to_host
from workloads.configs import ADAMW

pytestmark = pytest.mark.gpu
DEV = "cuda"


def unit_state(rng, plan):
    """fp32 master, zero m and v, bf16 parameter and R bf16 gradients."""
    full = rng.uniform(-0.5, 0.5, plan.T).astype(np.float32)
    master = torch.empty(plan.R * plan.S, device=DEV)
    F.fsdp_shard_pack(plan, to_dev(full), master)
    param = torch.empty(plan.R * plan.S, dtype=torch.bfloat16, device=DEV)
    F.fsdp_shard_pack(plan, to_dev(full), param)
    grads = [to_dev((rng.standard_normal(plan.T) * 1e-2).astype(np.float32)).bfloat16()
             for _ in range(plan.R)]
    return dict(master=master, m=torch.zeros_like(master), v=torch.zeros_like(master),
                param=param, grads=grads)


def clone_set(bufs):
    return {k: ([g.clone() for g in v] if isinstance(v, list) else v.clone())
            for k, v in bufs.items()}


def calls(p0, p1, rs, a, b, recv, red, moved, t):
    """The recorded sequence, bound to one set of buffers."""
    g0 = F.bind_gather_unflatten(p0, a["param"], recv[0])
    pair = F.bind_adamw_step_then_gather(p0, ADAMW, a["grads"], a["master"], a["m"], a["v"],
                                         a["param"], p1, b["param"], recv[1])
    step1 = F.bind_adamw_shard_step(p1, ADAMW, b["grads"], b["master"], b["m"], b["v"],
                                    b["param"])
    rsc = F.bind_reduce_scatter_avg(p1, b["grads"], red)

    def run():
        g0()
        pair(t)
        step1(t)
        rsc()
        F.fsdp_reshard(rs, a["master"], moved)
    return run


@pytest.mark.parametrize("R", [3, 8])
def test_captured_unit_loop_replays_match_eager_calls(R):
    print(f"[gpu] capture R={R}", flush=True)
    rng = np.random.default_rng(700 + R)
    p0 = F.Plan([(67, 5), (130,), (9, 4, 3)], R, "per_param")
    p1 = F.Plan([(200, 33), (7,)], R, "flat")
    p2 = F.Plan([(67, 5), (130,), (9, 4, 3)], R + 1, "flat")
    rs = F.Resharder(p0, p2)
    for p in (p0, p1, p2):
        p.prepare()                      # tables on the device before capture
    a, b = unit_state(rng, p0), unit_state(rng, p1)
    T = max(p0.T, p1.T)
    # a re-sharder uploads its table at its first call: make that call now
    F.fsdp_reshard(rs, a["master"], torch.empty((R + 1) * p2.S, device=DEV))

    def outputs():
        recv = [[torch.zeros(T, dtype=torch.bfloat16, device=DEV) for _ in range(R)]
                for _ in range(2)]
        return recv, torch.zeros(R * p1.S, device=DEV), torch.zeros((R + 1) * p2.S, device=DEV)

    # the captured set and the eager set start from the same contents
    ea, eb = clone_set(a), clone_set(b)
    recv, red, moved = outputs()
    erecv, ered, emoved = outputs()
    captured = calls(p0, p1, rs, a, b, recv, red, moved, t=2)
    eager = calls(p0, p1, rs, ea, eb, erecv, ered, emoved, t=2)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured()
    torch.cuda.synchronize()
    # capture records without running: the captured set is untouched
    assert_bitexact(to_host(a["master"]), to_host(ea["master"]), "before the first replay")

    noise = torch.randn(1 << 20, device=DEV)
    for k in range(1, 4):
        graph.replay()
        noise.mul_(0.5).add_(1.0)        # eager work of the program between replays
        eager()
        torch.cuda.synchronize()
        for name in ("master", "m", "v", "param"):
            assert_bitexact(to_host(a[name]), to_host(ea[name]), f"unit 0 {name}, replay {k}")
            assert_bitexact(to_host(b[name]), to_host(eb[name]), f"unit 1 {name}, replay {k}")
        for i in range(2):
            for r in range(R):
                assert_bitexact(to_host(recv[i][r]), to_host(erecv[i][r]),
                                f"receiver {i}.{r}, replay {k}")
        assert_bitexact(to_host(red), to_host(ered), f"reduce-scatter, replay {k}")
        assert_bitexact(to_host(moved), to_host(emoved), f"re-shard, replay {k}")
        print(f"[gpu] capture R={R} replay {k} ok", flush=True)
    # the replays did the work: the state moved and the receivers were filled
    assert np.any(to_host(a["m"]) != 0)
    assert np.any(to_host(recv[1][0]) != 0)
