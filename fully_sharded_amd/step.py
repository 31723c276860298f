"""The unit loop of one training step: for every FSDP unit in order, all-gather
+ unflatten its parameter shards, then the fused reduce-scatter-average +
AdamW + recast of its gradients ("FSDP Training Step Walkthrough", steps 1-6;
zwjcode FSDP2 page, section 05: one communication group per block).

Five schedules (and an automatic choice between two), same results bit for bit:
  serial    one stream: gather(u), step(u), gather(u+1), ...
  overlap   one stream: gather(0), then step(u) together with gather(u+1)
            (fsdp_adamw_step_then_gather: one launch for short steps), into
            two alternating receive buffers, then step(last) -- the
            prefetch of section 07 of the zwjcode FSDP2 page without a
            second stream.  With two gathers per step the forward gathers
            run unit by unit, and the backward goes from the last unit to
            the first: its re-gather, then step(u) together with the
            re-gather of unit u-1, then step(0)
  graph     the serial sequence recorded once as a HIP graph (StepGraph) and
            replayed each step with one launch
  graph-overlap  the overlap sequence (one gather per step) recorded as a
            HIP graph the same way
  auto      built like overlap; choose_schedule then times the overlap and
            serial sequences on the caller's own steps and keeps the faster
            (set_schedule switches between them at any step boundary)
  prefetch  gathers on their own stream run ahead of the steps, into two
            alternating receive buffers (zwjcode FSDP2 page, section 07:
            all-gather block k+1 while block k computes, at the price of a
            second receive buffer).  Unit u's gather waits for unit u's
            previous step (it reads the parameter that step writes) and unit
            u's step waits for its gather (it overwrites that parameter).

The runner only orders library calls on streams; every byte is moved by the
library's kernels.
"""

from __future__ import annotations

import ctypes

import torch

from .binding import (Plan, StepGraph, bind_adamw_shard_step, bind_adamw_step_then_gather,
                      bind_gather_unflatten)


class Unit:
    """Device buffers of one FSDP unit (all on the current GPU)."""

    def __init__(self, plan: Plan, master, m, v, param, grads):
        self.plan = plan
        self.master = master
        self.m = m
        self.v = v
        self.param = param
        self.grads = list(grads)


class StepRunner:
    """Runs training steps over a list of units.

    receivers: one list of R receiver tensors per receive buffer (at least
    as long as the largest unit); the prefetch and overlap schedules need
    two.
    gathers_per_step: 1 keeps the gathered parameters from forward to
    backward (reshard_after_forward=False), 2 frees them after forward and
    gathers again in backward (reshard_after_forward=True)."""

    def __init__(self, units, hp: dict, receivers, schedule: str = "serial",
                 gathers_per_step: int = 1):
        if schedule not in ("serial", "prefetch", "graph", "overlap", "graph-overlap", "auto"):
            raise ValueError(schedule)
        # "auto": the overlap schedule's resources (two receive buffers, the
        # paired calls), so that the serial and the overlap sequence can both
        # run; it starts as overlap
        self.switchable = ("overlap", "serial") if schedule == "auto" else (schedule,)
        if schedule == "auto":
            schedule = "overlap"
        if schedule == "graph-overlap" and gathers_per_step != 1:
            raise ValueError("the graph-overlap schedule gathers once per step")
        if schedule in ("prefetch", "overlap", "graph-overlap") and len(receivers) < 2:
            raise ValueError(f"the {schedule} schedule needs two receive buffers")
        if gathers_per_step not in (1, 2):
            raise ValueError("gathers_per_step is 1 or 2")
        self.units = list(units)
        self.schedule = schedule
        self.gathers_per_step = gathers_per_step
        nb = 2 if schedule in ("prefetch", "overlap", "graph-overlap") else 1
        self.calls = [(bind_gather_unflatten(u.plan, u.param, receivers[i % nb]),
                       bind_adamw_shard_step(u.plan, hp, u.grads, u.master, u.m, u.v, u.param))
                      for i, u in enumerate(self.units)]
        self.stream = torch.cuda.current_stream()
        self._hs = ctypes.c_void_p(self.stream.cuda_stream)
        if schedule in ("overlap", "graph-overlap"):
            us = self.units
            if gathers_per_step == 1:   # forward order: step u, gather u+1
                self.pairs = [bind_adamw_step_then_gather(
                    u.plan, hp, u.grads, u.master, u.m, u.v, u.param, us[i + 1].plan,
                    us[i + 1].param, receivers[(i + 1) % 2]) for i, u in enumerate(us[:-1])]
            else:                       # backward order: step u, re-gather u-1
                self.pairs = [bind_adamw_step_then_gather(
                    us[i].plan, hp, us[i].grads, us[i].master, us[i].m, us[i].v, us[i].param,
                    us[i - 1].plan, us[i - 1].param, receivers[(i - 1) % 2])
                    for i in range(len(us) - 1, 0, -1)]
        if schedule == "graph":
            self.graph = StepGraph(hp)
            for u in self.units:
                for _ in range(gathers_per_step):
                    self.graph.add_gather(u.plan, u.param, receivers[0])
                self.graph.add_adamw(u.plan, u.grads, u.master, u.m, u.v, u.param)
        if schedule == "graph-overlap":
            us = self.units
            self.graph = StepGraph(hp)
            self.graph.add_gather(us[0].plan, us[0].param, receivers[0])
            for i, u in enumerate(us[:-1]):
                self.graph.add_adamw_gather(u.plan, u.grads, u.master, u.m, u.v, u.param,
                                            us[i + 1].plan, us[i + 1].param,
                                            receivers[(i + 1) % 2])
            last = us[-1]
            self.graph.add_adamw(last.plan, last.grads, last.master, last.m, last.v, last.param)
        if schedule == "prefetch":
            self.s_gather = torch.cuda.Stream()   # default priority
            self.s_step = torch.cuda.Stream()
            self._hg = ctypes.c_void_p(self.s_gather.cuda_stream)
            self._hf = ctypes.c_void_p(self.s_step.cuda_stream)
            self.gathered = [torch.cuda.Event() for _ in self.units]
            self.stepped = [torch.cuda.Event() for _ in self.units]
            for e in self.stepped:
                e.record(self.stream)

    def step(self, t: int) -> None:
        """One training step with AdamW step counter t (>= 1), enqueued on
        the current stream (the prefetch schedule joins its streams back to
        it before returning)."""
        if self.schedule in ("graph", "graph-overlap"):
            self.graph.launch(t, self._hs)
            return
        if self.schedule == "overlap":
            if self.gathers_per_step == 1:
                self.calls[0][0](self._hs)
                for pair in self.pairs:
                    pair(t, self._hs)
                self.calls[-1][1](t, self._hs)
            else:
                for gather, _ in self.calls:      # forward
                    gather(self._hs)
                self.calls[-1][0](self._hs)       # backward: last unit first
                for pair in self.pairs:
                    pair(t, self._hs)
                self.calls[0][1](t, self._hs)
            return
        if self.schedule == "serial":
            for gather, fused in self.calls:
                for _ in range(self.gathers_per_step):
                    gather(self._hs)
                fused(t, self._hs)
            return
        start = torch.cuda.Event()
        start.record(self.stream)
        self.s_gather.wait_event(start)
        self.s_step.wait_event(start)
        for u, (gather, fused) in enumerate(self.calls):
            self.s_gather.wait_event(self.stepped[u])
            for _ in range(self.gathers_per_step):
                gather(self._hg)
            self.gathered[u].record(self.s_gather)
            self.s_step.wait_event(self.gathered[u])
            fused(t, self._hf)
            self.stepped[u].record(self.s_step)
        self.stream.wait_stream(self.s_gather)
        self.stream.wait_stream(self.s_step)

    def set_schedule(self, schedule: str) -> None:
        """Switch between the sequences the runner was built for (an "auto"
        runner: "overlap" and "serial"), at a step boundary."""
        if schedule not in self.switchable:
            raise ValueError(f"{schedule} is not one of {self.switchable}")
        self.schedule = schedule

    def memory_ledger(self, param_bytes: int = 2) -> dict:
        """Bytes one rank holds ("FSDP2 ... memory peak", section 01): its
        sharded state (16 per shard element per unit), the largest unsharded
        group while gathered, and, for the prefetch schedule, the next
        group's receive buffer (prefetch and overlap schedules); activations
        and temporaries excluded."""
        shard = sum(u.plan.state_bytes_per_rank() for u in self.units)
        largest = max(u.plan.T for u in self.units) * param_bytes
        two = self.schedule in ("prefetch", "overlap", "graph-overlap") or len(self.switchable) > 1
        prefetch = largest if two and len(self.units) > 1 else 0
        return dict(sharded_state=shard, largest_unsharded_group=largest, prefetch=prefetch,
                    peak_lower_bound=shard + largest + prefetch)


def choose_schedule(runners, step, candidates=("overlap", "serial"), steps: int = 20,
                    rounds: int = 3) -> dict:
    """Time each candidate schedule on `step` (a callable running one
    training step over `runners`, e.g. cycling buffer copies) for `steps`
    steps, in `rounds` alternating rounds on the current stream, and switch
    every runner to the fastest by median.  Every candidate gives the same
    results bit for bit, so the steps run here are ordinary training steps.
    Returns {"chosen": name, "ms_per_step": {name: [round times]}}."""
    stream = torch.cuda.current_stream()
    times = {c: [] for c in candidates}
    for _ in range(rounds):
        for c in candidates:
            for r in runners:
                r.set_schedule(c)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(steps):
                step()
            b.record(stream)
            torch.cuda.synchronize()
            times[c].append(a.elapsed_time(b) / steps)
    med = {c: sorted(v)[len(v) // 2] for c, v in times.items()}
    chosen = min(candidates, key=lambda c: med[c])
    for r in runners:
        r.set_schedule(chosen)
    return {"chosen": chosen, "ms_per_step": times}
