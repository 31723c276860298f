"""The unit loop's schedules give the same state bit for bit: the prefetch
schedule (gathers on their own stream, double receive buffer), two gathers
per step, and the step graph (the serial sequence replayed as one HIP graph)
change ordering, traffic or launch count, not results."""

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
    pdt = torch.bfloat16 if wl["param_dtype"] == "bf16" else torch.float32
    units = []
    for u in range(n_units or len(wl["units"])):
        full = gen.device_master(wl, u, shapes, DEV)
        master = torch.empty(R * pl.S, device=DEV)
        F.fsdp_shard_pack(pl, full, master)
        param = torch.empty(R * pl.S, dtype=pdt, device=DEV)
        F.fsdp_shard_pack(pl, full, param)
        grads = [gen.device_grad(wl, 1, u, r, pl.T, DEV) for r in range(R)]
        units.append(Unit(pl, master, torch.zeros_like(master), torch.zeros_like(master),
                          param, grads))
    recv = [[torch.empty(pl.T, dtype=pdt, device=DEV) for _ in range(R)]
            for _ in range(2)]
    return units, recv


def state_of(units):
    return [(u.master.clone(), u.m.clone(), u.v.clone(), bits(u.param)) for u in units]


def bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).clone()


@pytest.mark.parametrize("schedule,gathers", [("prefetch", 1), ("serial", 2), ("prefetch", 2),
                                              ("overlap", 1), ("overlap", 2)])
def test_schedules_agree_bit_for_bit(schedule, gathers):
    print(f"[gpu] schedule={schedule} gathers={gathers}", flush=True)
    ref_units, ref_recv = build("model12_r8")
    ref = StepRunner(ref_units, ADAMW, ref_recv, "serial", 1)
    units, recv = build("model12_r8")
    run = StepRunner(units, ADAMW, recv, schedule, gathers)
    before = None
    for t in (1, 2, 3):
        if t == 3:   # the parameters the last step's gathers read
            before = [u.param.clone() for u in ref_units[:2]]
        ref.step(t)
        run.step(t)
    torch.cuda.synchronize()
    for a, b in zip(state_of(ref_units), state_of(units)):
        for x, y in zip(a, b):
            assert torch.equal(x, y)
    # the receive buffers hold the last gathered units, the same in both runs
    n = len(units)
    if schedule == "overlap" and gathers == 2:
        # the backward runs from the last unit to the first: the last
        # re-gathers are those of units 1 and 0 (buffers 1 and 0), each
        # taken before that unit's step
        for b, p in enumerate(before):
            want = [torch.empty_like(x) for x in ref_recv[0]]
            F.fsdp_gather_unflatten(ref_units[b].plan, p, want)
            torch.cuda.synchronize()
            for r in range(len(want)):
                assert torch.equal(recv[b][r].view(torch.int16), want[r].view(torch.int16))
        return
    last = recv[(n - 1) % 2] if schedule in ("prefetch", "overlap") else recv[0]
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


@pytest.mark.parametrize("wl_name,gathers", [("model12_r8", 1), ("model12_r8", 2),
                                             ("block512_r3", 1), ("block512_flat_r3", 1),
                                             ("toy_2layer_r2", 1)])
def test_step_graph_replays_match_the_stream_calls(wl_name, gathers):
    """Every replay of the step graph, with unrelated eager work and a
    synchronisation between replays, leaves the state and the receive buffer
    bit-identical to the same step made with stream calls."""
    print(f"[gpu] step graph {wl_name} gathers={gathers}", flush=True)
    ref_units, ref_recv = build(wl_name)
    ref = StepRunner(ref_units, ADAMW, ref_recv, "serial", gathers)
    units, recv = build(wl_name)
    run = StepRunner(units, ADAMW, recv, "graph", gathers)
    n_nodes, n_adamw = run.graph.info()
    assert n_adamw == len(units) and n_nodes == len(units) * (gathers + 1)
    scratch = torch.randn(1 << 20, device=DEV)
    for t in (1, 2, 3, 4):
        run.step(t)
        scratch.mul_(1.0001).add_(1.0)            # the program's own eager work
        ref.step(t)
        torch.cuda.synchronize()
        for a, b in zip(state_of(ref_units), state_of(units)):
            for x, y in zip(a, b):
                assert torch.equal(x, y), f"step {t}"
        for r in range(len(recv[0])):
            assert torch.equal(bits(recv[0][r]), bits(ref_recv[0][r])), f"step {t}"


def test_step_graph_steps_need_not_be_consecutive():
    """The step counter comes from each launch: replaying t = 5 after t = 1
    matches the stream calls made with t = 1 then t = 5."""
    ref_units, ref_recv = build("block512_r4")
    units, recv = build("block512_r4")
    ref = StepRunner(ref_units, ADAMW, ref_recv, "serial")
    run = StepRunner(units, ADAMW, recv, "graph")
    for t in (1, 5, 2):
        ref.step(t)
        run.step(t)
    torch.cuda.synchronize()
    for a, b in zip(state_of(ref_units), state_of(units)):
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_step_graph_launches_on_alternating_streams():
    """Consecutive replays enqueued on two streams, with no host
    synchronisation between them: each launch on another stream waits for
    the previous replay (both read the graph's one record of AdamW
    scalars), so the state matches the stream calls bit for bit."""
    print("[gpu] step graph on alternating streams", flush=True)
    ref_units, ref_recv = build("model12_r8")
    units, recv = build("model12_r8")
    ref = StepRunner(ref_units, ADAMW, ref_recv, "serial")
    run = StepRunner(units, ADAMW, recv, "graph")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    torch.cuda.synchronize()
    for t in range(1, 7):
        run.graph.launch(t, streams[t % 2])
        ref.step(t)
    torch.cuda.synchronize()
    for a, b in zip(state_of(ref_units), state_of(units)):
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_step_graph_errors():
    units, recv = build("block512_r4")
    u = units[0]
    with pytest.raises(F.FsdpError):            # eps must be > 0
        F.StepGraph(dict(ADAMW, eps=0.0))
    g = F.StepGraph(ADAMW)
    g.launch(1)                                  # empty: nothing to run
    with pytest.raises(F.FsdpError):            # the parameter overlaps the master
        g.add_adamw(u.plan, u.grads, u.master, u.m, u.v, u.master.view(torch.bfloat16)[: u.param.numel()])
    g.add_gather(u.plan, u.param, recv[0])
    g.add_adamw(u.plan, u.grads, u.master, u.m, u.v, u.param)
    with pytest.raises(F.FsdpError):            # step counter starts at 1
        g.launch(0)
    g.launch(1)
    with pytest.raises(F.FsdpError):            # sealed by its first launch
        g.add_gather(u.plan, u.param, recv[1])
    torch.cuda.synchronize()
    assert g.info() == (2, 1)


@pytest.mark.parametrize("wl_name", ["toy_2layer_r2", "model12_flat_r8", "model12_perparam_r8"])
def test_overlap_schedule_other_workloads(wl_name):
    """The overlap schedule (each unit's step sharing its launch with the
    next unit's gather) against the serial one: fp32 toy, FlatParameter
    units, and 96 one-parameter units (ragged pieces, 3-element norms)."""
    print(f"[gpu] overlap {wl_name}", flush=True)
    ref_units, ref_recv = build(wl_name)
    ref = StepRunner(ref_units, ADAMW, ref_recv, "serial")
    units, recv = build(wl_name)
    run = StepRunner(units, ADAMW, recv, "overlap")
    for t in (1, 2, 3):
        ref.step(t)
        run.step(t)
    torch.cuda.synchronize()
    for a, b in zip(state_of(ref_units), state_of(units)):
        for x, y in zip(a, b):
            assert torch.equal(x, y)


@pytest.mark.parametrize("wl_name", ["toy_2layer_r2", "model12_flat_r8"])
def test_overlap_schedule_with_two_gathers(wl_name):
    """reshard_after_forward=True under the overlap schedule: forward
    gathers, then the backward from the last unit, each step paired with the
    re-gather of the unit before it; the same state as the serial loop."""
    ref_units, ref_recv = build(wl_name)
    ref = StepRunner(ref_units, ADAMW, ref_recv, "serial", 2)
    units, recv = build(wl_name)
    run = StepRunner(units, ADAMW, recv, "overlap", 2)
    for t in (1, 2, 3):
        ref.step(t)
        run.step(t)
    torch.cuda.synchronize()
    for a, b in zip(state_of(ref_units), state_of(units)):
        for x, y in zip(a, b):
            assert torch.equal(x, y)


@pytest.mark.parametrize("wl_name", ["model12_r8", "toy_2layer_r2", "model12_pair_r8"])
def test_graph_overlap_replays_match_the_overlap_calls(wl_name):
    """The overlap sequence recorded as a step graph (paired nodes): every
    replay, with eager work and a synchronisation between replays, leaves
    the same bits as the stream calls of the overlap schedule."""
    print(f"[gpu] graph-overlap {wl_name}", flush=True)
    ref_units, ref_recv = build(wl_name)
    ref = StepRunner(ref_units, ADAMW, ref_recv, "overlap")
    units, recv = build(wl_name)
    run = StepRunner(units, ADAMW, recv, "graph-overlap")
    n_nodes, n_adamw = run.graph.info()
    assert n_adamw == len(units)
    scratch = torch.randn(1 << 20, device=DEV)
    for t in (1, 2, 3):
        run.step(t)
        scratch.mul_(0.999).add_(1.0)
        ref.step(t)
        torch.cuda.synchronize()
        for a, b in zip(state_of(ref_units), state_of(units)):
            for x, y in zip(a, b):
                assert torch.equal(x, y), f"step {t}"
        for k in range(2):
            for r in range(len(recv[k])):
                assert torch.equal(bits(recv[k][r]), bits(ref_recv[k][r])), f"step {t}"


def test_units_sharing_a_plan_on_two_streams():
    """Operations with the same plan on two streams at once (the plan's work
    tables are shared): each unit ends bit-identical to the serial run."""
    ref_units, ref_recv = build("model12_r8", n_units=4)
    ref = StepRunner(ref_units, ADAMW, ref_recv, "serial")
    units, recv = build("model12_r8", n_units=4)
    assert units[0].plan is units[3].plan
    other = [[torch.empty_like(x) for x in recv[0]] for _ in range(2)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        a = StepRunner(units[:2], ADAMW, recv, "overlap")
    with torch.cuda.stream(s2):
        b = StepRunner(units[2:], ADAMW, other, "serial")
    assert a.stream == s1 and b.stream == s2
    for t in (1, 2, 3):
        ref.step(t)
        a.step(t)
        b.step(t)
    torch.cuda.synchronize()
    for x, y in zip(state_of(ref_units), state_of(units)):
        for p, q in zip(x, y):
            assert torch.equal(p, q)


def build_wide(R, layout, n_units, seed):
    """n_units units of ragged shapes sharing one plan at a world size above
    8 (the kernels with 64 pointer slots), bf16 parameters and gradients."""
    gen_ = torch.Generator(device=DEV)
    gen_.manual_seed(seed)
    pl = F.Plan([(2 * R + 3, 5), (R - 1,), (7, 3, 2)], R, layout)
    units = []
    for _ in range(n_units):
        full = torch.rand(pl.T, generator=gen_, device=DEV).sub_(0.5)
        master = torch.empty(R * pl.S, device=DEV)
        F.fsdp_shard_pack(pl, full, master)
        param = torch.empty(R * pl.S, dtype=torch.bfloat16, device=DEV)
        F.fsdp_shard_pack(pl, full, param)
        grads = [torch.randn(pl.T, generator=gen_, device=DEV).mul_(1e-2).bfloat16()
                 for _ in range(R)]
        units.append(Unit(pl, master, torch.zeros_like(master), torch.zeros_like(master),
                          param, grads))
    recv = [[torch.empty(pl.T, dtype=torch.bfloat16, device=DEV) for _ in range(R)]
            for _ in range(2)]
    return units, recv


@pytest.mark.parametrize("R,layout,schedule,ref_schedule", [
    (13, "per_param", "graph", "serial"), (64, "flat", "graph", "serial"),
    (13, "flat", "graph-overlap", "overlap"), (64, "per_param", "graph-overlap", "overlap")])
def test_step_graph_at_world_sizes_above_eight(R, layout, schedule, ref_schedule):
    """The step graph with the generic kernels (R > 8, 64 pointer slots):
    every replay, with eager work and a synchronisation between replays,
    matches the stream calls of the same schedule bit for bit."""
    print(f"[gpu] step graph R={R} {layout} {schedule}", flush=True)
    ref_units, ref_recv = build_wide(R, layout, 3, seed=R)
    ref = StepRunner(ref_units, ADAMW, ref_recv, ref_schedule)
    units, recv = build_wide(R, layout, 3, seed=R)
    run = StepRunner(units, ADAMW, recv, schedule)
    assert run.graph.info()[1] == len(units)
    scratch = torch.randn(1 << 16, device=DEV)
    for t in (1, 2, 3):
        run.step(t)
        scratch.mul_(0.5).add_(1.0)
        ref.step(t)
        torch.cuda.synchronize()
        for a, b in zip(state_of(ref_units), state_of(units)):
            for x, y in zip(a, b):
                assert torch.equal(x, y), f"step {t}"
        n_buf = 2 if schedule == "graph-overlap" else 1
        for k in range(n_buf):
            for r in range(R):
                assert torch.equal(bits(recv[k][r]), bits(ref_recv[k][r])), f"step {t}"
    # the replays did the work
    assert bool((units[0].m != 0).any())


@pytest.mark.parametrize("gathers", [1, 2])
def test_auto_schedule_choice_and_switching_keep_the_results(gathers):
    """An "auto" runner: choose_schedule times the overlap and serial
    sequences on ordinary steps and keeps the faster; switching between them
    at step boundaries leaves the state bit-identical to serial steps (with
    two gathers per step the overlap sequence runs the backward from the
    last unit)."""
    from fully_sharded_amd.step import choose_schedule
    print(f"[gpu] auto schedule, {gathers} gathers", flush=True)
    ref_units, ref_recv = build("model12_r8", n_units=4)
    ref = StepRunner(ref_units, ADAMW, ref_recv, "serial", gathers)
    units, recv = build("model12_r8", n_units=4)
    run = StepRunner(units, ADAMW, recv, "auto", gathers)
    assert run.schedule == "overlap"
    with pytest.raises(ValueError):
        run.set_schedule("prefetch")
    t = [0]

    def step():
        t[0] += 1
        run.step(t[0])

    info = choose_schedule([run], step, steps=2, rounds=2)
    assert info["chosen"] in ("overlap", "serial") and run.schedule == info["chosen"]
    assert all(len(v) == 2 and min(v) > 0 for v in info["ms_per_step"].values())
    run.set_schedule("serial")
    step()
    run.set_schedule("overlap")
    step()
    assert t[0] == 10
    for s in range(1, t[0] + 1):
        ref.step(s)
    torch.cuda.synchronize()
    for a, b in zip(state_of(ref_units), state_of(units)):
        for x, y in zip(a, b):
            assert torch.equal(x, y)
    led = run.memory_ledger()
    assert led["prefetch"] == 2 * units[0].plan.T
