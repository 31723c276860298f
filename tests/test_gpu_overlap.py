"""fsdp_adamw_step_then_gather: the fused AdamW step of one unit enqueued
together with the all-gather of the next unit (FSDP's prefetch).  Steps of
up to 65,536 work items share one launch with the gather, longer ones take
two; both give the bits of the two separate calls, and the oracle's
results."""

import numpy as np
import pytest
import torch

import fully_sharded_amd as F
from oracle import fsdp_oracle as O
from tests.gpu_util import (assert_adamw_close, assert_bitexact, to_dev, to_host)
from workloads.configs import ADAMW, BLOCK_512, LINEARS_512, shapes_of

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    F.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class HostUnit:
    """Seeded host state of one unit: fp32 master shards (m = v = 0), the
    parameter shards, R gradient replicas."""

    def __init__(self, shapes, R, layout, seed, pdt="bf16", gdt="bf16"):
        self.po = O.plan_layout(shapes, R, layout)
        self.pl = F.Plan(shapes, R, layout)
        rng = np.random.default_rng(seed)
        full = rng.uniform(-0.05, 0.05, self.po.T).astype(np.float32)
        self.master = O.shard_pack(self.po, full)
        self.m = np.zeros_like(self.master)
        self.v = np.zeros_like(self.master)
        self.param = O.bf16_rne(self.master) if pdt == "bf16" else self.master.copy()
        g = [(rng.standard_normal(self.po.T) * 1e-3).astype(np.float32) for _ in range(R)]
        self.grads = [O.bf16_rne(x) for x in g] if gdt == "bf16" else g
        self.pdt = pdt

    def device(self):
        d = dict(master=to_dev(self.master.reshape(-1)), m=to_dev(self.m.reshape(-1)),
                 v=to_dev(self.v.reshape(-1)), param=to_dev(self.param.reshape(-1)),
                 grads=[to_dev(x) for x in self.grads])
        return d


def receivers(pl, dtype, n=None):
    return [torch.full((pl.T,), 3, dtype=dtype, device=DEV) for _ in range(n or pl.R)]


def run_both(a: HostUnit, b: HostUnit, steps=(1, 2)):
    """Runs the pair call and the two separate calls on copies of the same
    state; returns both sets of device results."""
    out = []
    for combined in (True, False):
        da, db = a.device(), b.device()
        tdt = da["param"].dtype
        recv = receivers(b.pl, tdt)
        for t in steps:
            if combined:
                F.fsdp_adamw_step_then_gather(a.pl, ADAMW, t, da["grads"], da["master"], da["m"],
                                              da["v"], da["param"], b.pl, db["param"], recv)
            else:
                F.fsdp_adamw_shard_step(a.pl, ADAMW, t, da["grads"], da["master"], da["m"],
                                        da["v"], da["param"])
                F.fsdp_gather_unflatten(b.pl, db["param"], recv)
        torch.cuda.synchronize()
        out.append((da, recv))
    return out


def assert_same(x, y):
    for k in ("master", "m", "v", "param"):
        assert_bitexact(to_host(x[0][k]), to_host(y[0][k]), k)
    for r, (p, q) in enumerate(zip(x[1], y[1])):
        assert_bitexact(to_host(p), to_host(q), f"receiver {r}")


@pytest.mark.parametrize("case", ["short_bf16", "short_ragged_r3", "short_fp32", "capped_pair",
                                  "capped_pair_flat", "short_mixed_world", "mixed_world_wide",
                                  "wide_world", "f32_grads_bf16_params", "f32_params_r8",
                                  "flat_r16", "odd_pieces_r9"])
def test_pair_equals_the_two_calls(case):
    print(f"[gpu] step_then_gather {case}", flush=True)
    blk, lin = shapes_of(BLOCK_512), shapes_of(LINEARS_512)
    if case == "short_bf16":          # one launch; the next unit has another plan
        a, b = HostUnit(blk, 4, "per_param", 1), HostUnit(lin, 4, "flat", 2)
    elif case == "short_ragged_r3":   # padding, misaligned gradient sources
        a, b = HostUnit(blk, 3, "per_param", 3), HostUnit(blk, 3, "flat", 4)
    elif case == "short_fp32":        # fp32 gradients and parameters (4-byte gather)
        a = HostUnit([(37, 5), (11,)], 2, "per_param", 5, pdt="f32", gdt="f32")
        b = HostUnit([(9, 7), (3,)], 2, "per_param", 6, pdt="f32", gdt="f32")
    elif case == "short_mixed_world":  # the two halves of one launch with different R
        a, b = HostUnit(blk, 3, "per_param", 11), HostUnit(lin, 8, "flat", 12)
    elif case == "mixed_world_wide":  # R <= 8 step, R > 8 gather: two launches
        a, b = HostUnit(blk, 4, "per_param", 13), HostUnit(lin, 16, "flat", 14)
    elif case == "wide_world":        # R > 8 on both halves: one launch, 64 slots
        a, b = HostUnit([(300, 40), (50,)], 12, "per_param", 15), HostUnit(lin, 9, "flat", 16)
    elif case == "f32_grads_bf16_params":  # e.g. accumulated fp32 gradients
        a = HostUnit(blk, 8, "per_param", 17, pdt="bf16", gdt="f32")
        b = HostUnit(blk, 8, "per_param", 18)
    elif case == "f32_params_r8":     # fp32 parameters, scattered windows at R = 8
        a = HostUnit(blk, 8, "per_param", 19, pdt="f32")
        b = HostUnit(lin, 8, "per_param", 21, pdt="f32")
    elif case == "flat_r16":          # R > 8, every item even: adjacent pairs, 64 slots
        a, b = HostUnit(lin, 16, "flat", 22), HostUnit(blk, 16, "per_param", 23)
    elif case == "odd_pieces_r9":     # R = 9: even pieces and odd LayerNorm pieces in one step
        a, b = HostUnit(blk, 9, "per_param", 24), HostUnit(lin, 9, "flat", 25)
    elif case == "capped_pair":       # > 4,096 work items: one launch, 4 per CU
        a, b = HostUnit(blk * 2, 8, "per_param", 7), HostUnit(blk, 8, "per_param", 8)
    else:                             # capped_pair_flat
        a, b = HostUnit(blk * 2, 8, "flat", 9), HostUnit(lin * 2, 8, "flat", 10)
    pair, sep = run_both(a, b)
    assert_same(pair, sep)
    # and the oracle: two steps of unit a, the gather of unit b
    mo, mm, vv = a.master, a.m, a.v
    for t in (1, 2):
        mo, mm, vv, _ = O.shard_step(a.po, a.grads, mo, mm, vv, t, ADAMW, a.pdt)
    assert_adamw_close(to_host(pair[0]["master"]).reshape(a.po.R, a.po.S), mo, "master")
    assert_adamw_close(to_host(pair[0]["m"]).reshape(a.po.R, a.po.S), mm, "m")
    assert_adamw_close(to_host(pair[0]["v"]).reshape(a.po.R, a.po.S), vv, "v")
    full, _ = O.gather_unflatten(b.po, b.param)
    for r in pair[1]:
        assert_bitexact(to_host(r), full, "gather")


def test_skipped_receivers_and_no_receivers():
    blk = shapes_of(BLOCK_512)
    a, b = HostUnit(blk, 4, "per_param", 11), HostUnit(blk, 4, "per_param", 12)
    da, db = a.device(), b.device()
    recv = receivers(b.pl, torch.bfloat16)
    some = [recv[0], None, recv[2], None]
    F.fsdp_adamw_step_then_gather(a.pl, ADAMW, 1, da["grads"], da["master"], da["m"], da["v"],
                                  da["param"], b.pl, db["param"], some)
    torch.cuda.synchronize()
    full, _ = O.gather_unflatten(b.po, b.param)
    assert_bitexact(to_host(recv[0]), full, "receiver 0")
    assert_bitexact(to_host(recv[2]), full, "receiver 2")
    assert (recv[1] == 3).all() and (recv[3] == 3).all()   # skipped: untouched
    # no receiver at all: only the step runs
    dc = a.device()
    F.fsdp_adamw_step_then_gather(a.pl, ADAMW, 1, dc["grads"], dc["master"], dc["m"], dc["v"],
                                  dc["param"], b.pl, db["param"], [None] * 4)
    torch.cuda.synchronize()
    assert_bitexact(to_host(dc["master"]), to_host(da["master"]), "step only")


def test_pair_rejects_memory_the_two_share():
    blk = shapes_of(BLOCK_512)
    a, b = HostUnit(blk, 4, "per_param", 13), HostUnit(blk, 4, "per_param", 14)
    da, db = a.device(), b.device()
    recv = receivers(b.pl, torch.bfloat16)
    T = b.pl.T
    args = (a.pl, ADAMW, 1, da["grads"], da["master"], da["m"], da["v"], da["param"], b.pl)
    with pytest.raises(F.FsdpError):     # a receiver inside the master
        bad = [da["master"].view(torch.bfloat16)[:T]] + recv[1:]
        F.fsdp_adamw_step_then_gather(*args, db["param"], bad)
    with pytest.raises(F.FsdpError):     # a receiver inside a gradient replica
        F.fsdp_adamw_step_then_gather(*args, db["param"], [da["grads"][1]] + recv[1:])
    with pytest.raises(F.FsdpError):     # the gather reads what the step writes
        F.fsdp_adamw_step_then_gather(*args, da["param"], recv)
    with pytest.raises(F.FsdpError):     # step counter starts at 1
        F.fsdp_adamw_step_then_gather(a.pl, ADAMW, 0, da["grads"], da["master"], da["m"],
                                      da["v"], da["param"], b.pl, db["param"], recv)
    torch.cuda.synchronize()
    assert (recv[0] == 3).all()          # nothing was enqueued


@pytest.mark.parametrize("R", [8, 16])
def test_specials_through_the_paired_step(R):
    """NaN, +-Inf, -0 and overflow in the gradients of the step half of the
    paired launch, in a rank's even piece of the first parameter (adjacent
    element pairs) and in the 1-element pieces of the second (the strided
    form): master, m, v and the parameter equal the oracle's bit for bit,
    NaN compared by class; the gather half equals the oracle's gather."""
    print(f"[gpu] step_then_gather specials R={R}", flush=True)
    shapes = [(2 * R, 6), (R // 2,)]
    po = O.plan_layout(shapes, R, O.PER_PARAM)
    pl = F.Plan(shapes, R, O.PER_PARAM)
    T, S = po.T, po.S
    rng = np.random.default_rng(300 + R)
    grads = [(rng.standard_normal(T) * 1e-3).astype(np.float32) for _ in range(R)]
    w0 = 12 * R                    # the second parameter's first element
    for base in (0, w0):
        for g in grads:
            g[base] = -0.0
        grads[0][base + 1] = np.nan
        grads[1][base + 2], grads[2][base + 2] = np.inf, -np.inf
        grads[3][base + 3] = np.inf
    for g in grads:
        g[4] = 3.0e38
    grads[0][5] = -0.0
    grads = [O.bf16_rne(g) for g in grads]
    master = O.shard_pack(po, rng.uniform(-1, 1, T).astype(np.float32))
    master[0, 0] = -0.0
    nb = HostUnit([(33, 4), (5,)], R, "flat", 60 + R)
    md = to_dev(master.reshape(-1))
    m_d, v_d = torch.zeros_like(md), torch.zeros_like(md)
    pd = torch.empty(R * S, dtype=torch.bfloat16, device=DEV)
    recv = receivers(nb.pl, torch.bfloat16)
    F.fsdp_adamw_step_then_gather(pl, ADAMW, 1, [to_dev(g) for g in grads], md, m_d, v_d, pd,
                                  nb.pl, to_dev(nb.param.reshape(-1)), recv)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        mo, mm, vv, pp = O.shard_step(po, grads, master, np.zeros_like(master),
                                      np.zeros_like(master), 1, ADAMW, "bf16")
    for got, want, name in ((to_host(md).reshape(R, S), mo, "master"),
                            (to_host(m_d).reshape(R, S), mm, "m"),
                            (to_host(v_d).reshape(R, S), vv, "v")):
        nan = np.isnan(want)
        assert nan.any() or name != "master"
        assert np.array_equal(np.isnan(got), nan), name
        assert_bitexact(np.where(nan, 0, got), np.where(nan, 0, want), name)
    gq = to_host(pd).reshape(R, S)
    qnan = (pp & 0x7FFF) > 0x7F80
    assert np.array_equal((gq & 0x7FFF) > 0x7F80, qnan)
    assert_bitexact(np.where(qnan, 0, gq), np.where(qnan, 0, pp), "param")
    full, _ = O.gather_unflatten(nb.po, nb.param)
    for r in recv:
        assert_bitexact(to_host(r), full, "gather")


def test_pair_with_bases_off_alignment():
    """The paired call at R = 8 with the step's arrays a few elements past
    16-byte alignment: every item takes the two strided elements instead of
    the adjacent pairs; bit for bit against the oracle."""
    print("[gpu] step_then_gather, bases off alignment", flush=True)
    blk, lin = shapes_of(BLOCK_512), shapes_of(LINEARS_512)
    a, b = HostUnit(blk, 8, "per_param", 26), HostUnit(lin, 8, "flat", 27)

    def place(x: np.ndarray, k: int):
        t = to_dev(x.reshape(-1))
        base = torch.empty(t.numel() + 8, dtype=t.dtype, device=DEV)
        base[k:k + t.numel()].copy_(t)
        return base[k:k + t.numel()]

    md, m_d, v_d = place(a.master, 1), place(a.m, 3), place(a.v, 1)
    pd = place(a.param, 1)
    g_d = [place(g, 1 + q % 3) for q, g in enumerate(a.grads)]
    recv = receivers(b.pl, torch.bfloat16)
    nparam = to_dev(b.param.reshape(-1))
    mo, mm, vv = a.master, a.m, a.v
    for t in (1, 2):
        F.fsdp_adamw_step_then_gather(a.pl, ADAMW, t, g_d, md, m_d, v_d, pd, b.pl, nparam, recv)
        mo, mm, vv, pp = O.shard_step(a.po, a.grads, mo, mm, vv, t, ADAMW, "bf16")
    torch.cuda.synchronize()
    R, S = a.po.R, a.po.S
    assert_bitexact(to_host(md).reshape(R, S), mo, "master")
    assert_bitexact(to_host(m_d).reshape(R, S), mm, "m")
    assert_bitexact(to_host(v_d).reshape(R, S), vv, "v")
    assert_bitexact(to_host(pd).reshape(R, S), pp, "param")
    full, _ = O.gather_unflatten(b.po, b.param)
    for r in recv:
        assert_bitexact(to_host(r), full, "gather")


@pytest.mark.parametrize("R", [1, 2, 64])
def test_pair_at_extreme_world_sizes(R):
    """One rank (the step is local, the gather a copy) and 64 ranks (most
    ranks own no rows of the small parameters): the pair call equals the two
    calls and the oracle."""
    print(f"[gpu] step_then_gather R={R}", flush=True)
    shapes = [(65, 9), (7,), (130, 3)]
    a = HostUnit(shapes, R, "per_param", 20 + R)
    b = HostUnit([(33, 4), (5,)], R, "flat", 40 + R)
    pair, sep = run_both(a, b)
    assert_same(pair, sep)
    mo, mm, vv = a.master, a.m, a.v
    for t in (1, 2):
        mo, mm, vv, _ = O.shard_step(a.po, a.grads, mo, mm, vv, t, ADAMW, a.pdt)
    assert_adamw_close(to_host(pair[0]["master"]).reshape(a.po.R, a.po.S), mo, "master")
    full, _ = O.gather_unflatten(b.po, b.param)
    for r in pair[1]:
        assert_bitexact(to_host(r), full, "gather")


@pytest.mark.parametrize("hp,t", [
    (dict(lr=0.1, beta1=0.0, beta2=0.5, eps=1e-3, weight_decay=0.0), 1),
    (dict(lr=3e-4, beta1=0.95, beta2=0.9999, eps=1e-12, weight_decay=0.1), 1000),
    (dict(lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.5), 7),
    (dict(lr=1e-2, beta1=0.5, beta2=0.25, eps=1.0, weight_decay=1e-4), 100000),
])
def test_other_hyper_parameters_and_step_counters(hp, t):
    """The step's float64 scalars (decay, bias corrections at large t) for
    other hyper-parameters, through the stream call, the paired call and a
    step graph: each agrees with the oracle."""
    blk = shapes_of(BLOCK_512)
    a, b = HostUnit(blk, 4, "per_param", 31), HostUnit(blk, 4, "per_param", 32)
    mo, mm, vv, _ = O.shard_step(a.po, a.grads, a.master, a.m, a.v, t, hp, "bf16")
    outs = []
    for how in ("stream", "pair", "graph"):
        da, db = a.device(), b.device()
        recv = receivers(b.pl, torch.bfloat16)
        if how == "stream":
            F.fsdp_adamw_shard_step(a.pl, hp, t, da["grads"], da["master"], da["m"], da["v"],
                                    da["param"])
        elif how == "pair":
            F.fsdp_adamw_step_then_gather(a.pl, hp, t, da["grads"], da["master"], da["m"],
                                          da["v"], da["param"], b.pl, db["param"], recv)
        else:
            g = F.StepGraph(hp)
            g.add_adamw(a.pl, da["grads"], da["master"], da["m"], da["v"], da["param"])
            g.launch(t)
        torch.cuda.synchronize()
        outs.append(da)
        assert_adamw_close(to_host(da["master"]).reshape(a.po.R, a.po.S), mo, f"master {how}")
        assert_adamw_close(to_host(da["m"]).reshape(a.po.R, a.po.S), mm, f"m {how}")
        assert_adamw_close(to_host(da["v"]).reshape(a.po.R, a.po.S), vv, f"v {how}")
    for k in ("master", "m", "v", "param"):
        assert_bitexact(to_host(outs[1][k]), to_host(outs[0][k]), f"pair vs stream {k}")
        assert_bitexact(to_host(outs[2][k]), to_host(outs[0][k]), f"graph vs stream {k}")


def test_pair_long_steps_take_two_launches():
    """A step of more than 65,536 work items (70M elements at R = 8) runs
    in its own launch, then the gather: the same bits as the two calls."""
    R, T = 8, 70_000_000
    pa = F.Plan([(T,)], R, "flat")
    pb = F.Plan(shapes_of(BLOCK_512), R, "per_param")
    assert len(pa.work_items(0)) > 65536
    gen_ = torch.Generator(device=DEV).manual_seed(70)
    grads = [(torch.randn(T, device=DEV, generator=gen_) * 1e-2).to(torch.bfloat16)
             for _ in range(R)]
    master0 = torch.rand(R * pa.S, device=DEV, generator=gen_) - 0.5
    nparam = (torch.rand(R * pb.S, device=DEV, generator=gen_) - 0.5).to(torch.bfloat16)
    out = []
    for combined in (True, False):
        master, m, v = master0.clone(), torch.zeros_like(master0), torch.zeros_like(master0)
        param = master0.to(torch.bfloat16)
        recv = receivers(pb, torch.bfloat16)
        for t in (1, 2):
            if combined:
                F.fsdp_adamw_step_then_gather(pa, ADAMW, t, grads, master, m, v, param, pb,
                                              nparam, recv)
            else:
                F.fsdp_adamw_shard_step(pa, ADAMW, t, grads, master, m, v, param)
                F.fsdp_gather_unflatten(pb, nparam, recv)
        torch.cuda.synchronize()
        out.append((master, m, v, param, recv))
    for x, y in zip(out[0][:4], out[1][:4]):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)
    for p_, q_ in zip(out[0][4], out[1][4]):
        assert torch.equal(p_.view(torch.int16), q_.view(torch.int16))
