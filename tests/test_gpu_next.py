"""GPU parity of the widened rows against the oracle, through the C ABI:
re-sharding to another world size / layout (bit-exact), gradient
accumulation over micro-batches (bit-exact) feeding the fused step, and the
DDP all-reduce comparator (bit-exact)."""

import numpy as np
import pytest
import torch

import fully_sharded_amd as F
from oracle import fsdp_oracle as O
from tests.gpu_util import (assert_adamw_close, assert_bf16_within_ulp, assert_bitexact,
                            to_dev, to_host)
from workloads import gen
from workloads.configs import ADAMW, BLOCK_512, WORKLOADS, shapes_of

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


# ------------------------------------------------------------- reshard
@pytest.mark.parametrize("Ra,la,Rb,lb", [(8, "per_param", 4, "per_param"),
                                         (4, "per_param", 8, "flat"),
                                         (8, "flat", 3, "per_param"),
                                         (3, "per_param", 3, "flat")])
def test_reshard_block_state_bit_exact(Ra, la, Rb, lb):
    banner(f"reshard block R={Ra} {la} -> R={Rb} {lb}")
    shapes = shapes_of(BLOCK_512)
    pa, pb = O.plan_layout(shapes, Ra, la), O.plan_layout(shapes, Rb, lb)
    ga, gb = F.Plan(shapes, Ra, la), F.Plan(shapes, Rb, lb)
    rs = F.Resharder(ga, gb)
    rng = np.random.default_rng(Ra * 31 + Rb)
    for dt in ("f32", "bf16"):
        full = rng.standard_normal(pa.T).astype(np.float32)
        if dt == "bf16":
            full = O.bf16_rne(full)
        src_h = O.shard_pack(pa, full)
        src = to_dev(src_h.reshape(-1))
        dst = torch.full((Rb * pb.S,), 7, dtype=src.dtype, device=DEV)   # padding must be zeroed
        F.fsdp_reshard(rs, src, dst)
        assert_bitexact(to_host(dst).reshape(Rb, pb.S), O.reshard(pa, pb, src_h), f"reshard {dt}")


@pytest.mark.parametrize("Ra,Rb", [(1, 7), (5, 2), (13, 64), (64, 3)])
def test_reshard_ragged_shapes(Ra, Rb):
    rng = np.random.default_rng(Ra + 1000 * Rb)
    for trial in range(8):
        shapes = [(int(rng.integers(1, 3 * max(Ra, Rb) + 3)),) +
                  tuple(int(x) for x in rng.integers(1, 40, int(rng.integers(0, 3))))
                  for _ in range(int(rng.integers(1, 5)))]
        la = "flat" if trial % 2 else "per_param"
        lb = "per_param" if trial % 3 else "flat"
        pa, pb = O.plan_layout(shapes, Ra, la), O.plan_layout(shapes, Rb, lb)
        rs = F.Resharder(F.Plan(shapes, Ra, la), F.Plan(shapes, Rb, lb))
        src_h = O.shard_pack(pa, rng.integers(1, 2**31, pa.T).astype(np.uint32).view(np.float32))
        dst = torch.empty(Rb * pb.S, dtype=torch.float32, device=DEV)
        F.fsdp_reshard(rs, to_dev(src_h.reshape(-1)), dst)
        assert_bitexact(to_host(dst).reshape(Rb, pb.S), O.reshard(pa, pb, src_h), "reshard ragged")


def test_restore_at_another_world_size_then_step():
    """The 12-layer model's unit 0 trained 2 steps at R=8, its parameter,
    master, m and v re-sharded to R=4, one more step at R=4: the same state
    as the oracle stepping the full tensors (shard-wise AdamW is the slice
    of the full step)."""
    wl = WORKLOADS["model12_r8"]
    shapes = shapes_of(wl["units"][0])
    p8, p4 = O.plan_layout(shapes, 8, "per_param"), O.plan_layout(shapes, 4, "per_param")
    g8, g4 = F.Plan(shapes, 8, "per_param"), F.Plan(shapes, 4, "per_param")
    master_full = gen.host_master(wl, 0, shapes)
    md = torch.empty(8 * p8.S, device=DEV)
    F.fsdp_shard_pack(g8, to_dev(master_full), md)
    m = torch.zeros_like(md)
    v = torch.zeros_like(md)
    pd = torch.empty(8 * p8.S, dtype=torch.bfloat16, device=DEV)
    mo, mmo, vvo = master_full.copy(), np.zeros(p8.T, np.float32), np.zeros(p8.T, np.float32)
    for t in (1, 2):
        grads = [gen.host_grad(wl, t, 0, r, p8.T) for r in range(8)]
        F.fsdp_adamw_shard_step(g8, ADAMW, t, [to_dev(g) for g in grads], md, m, v, pd)
        mo, mmo, vvo = O.adamw_step(mo, mmo, vvo, O.rank_order_mean(grads), t, **ADAMW)
    rs = F.Resharder(g8, g4)
    new = {}
    for name, x in (("master", md), ("m", m), ("v", v), ("param", pd)):
        y = torch.empty(4 * p4.S, dtype=x.dtype, device=DEV)
        F.fsdp_reshard(rs, x, y)
        new[name] = y
    # a step at the new world size: 4 ranks' gradients (their mean is the
    # full-batch gradient of this step)
    grads4 = [gen.host_grad(wl, 3, 0, r, p4.T) for r in range(4)]
    F.fsdp_adamw_shard_step(g4, ADAMW, 3, [to_dev(g) for g in grads4], new["master"], new["m"],
                            new["v"], new["param"])
    mo, mmo, vvo = O.adamw_step(mo, mmo, vvo, O.rank_order_mean(grads4), 3, **ADAMW)
    assert_adamw_close(to_host(new["master"]).reshape(4, p4.S), O.shard_pack(p4, mo), "master")
    assert_adamw_close(to_host(new["m"]).reshape(4, p4.S), O.shard_pack(p4, mmo), "m")
    assert_adamw_close(to_host(new["v"]).reshape(4, p4.S), O.shard_pack(p4, vvo), "v")
    assert_bf16_within_ulp(to_host(new["param"]).reshape(4, p4.S),
                           O.bf16_rne(O.shard_pack(p4, mo)), "param")


# -------------------------------------------------- gradient accumulation
@pytest.mark.parametrize("name", ["block512_r4", "block512_r3", "toy_2layer_r2"])
def test_accumulate_then_fused_step(name):
    wl = WORKLOADS[name]
    R = wl["R"]
    shapes = shapes_of(wl["units"][0])
    po = O.plan_layout(shapes, R, wl["layout"])
    pg = F.Plan(shapes, R, wl["layout"])
    K = 3
    banner(f"accumulate {name} K={K}")
    micro = [[gen.host_grad(wl, 10 + k, 0, r, po.T) for r in range(R)] for k in range(K)]
    acc = [torch.full((po.T,), 3.0, device=DEV) for _ in range(R)]
    for k in range(K):
        F.fsdp_grad_accumulate(pg, [to_dev(g) for g in micro[k]], acc, first=(k == 0))
    want = [O.grad_accumulate([micro[k][r] for k in range(K)]) for r in range(R)]
    for r in range(R):
        assert_bitexact(to_host(acc[r]), want[r], f"acc rank {r}")
    master_full = gen.host_master(wl, 0, shapes)
    md = torch.empty(R * po.S, device=DEV)
    F.fsdp_shard_pack(pg, to_dev(master_full), md)
    m, v = torch.zeros_like(md), torch.zeros_like(md)
    pdt = torch.bfloat16 if wl["param_dtype"] == "bf16" else torch.float32
    pd = torch.empty(R * po.S, dtype=pdt, device=DEV)
    F.fsdp_adamw_shard_step(pg, ADAMW, 1, acc, md, m, v, pd)
    mo = O.shard_pack(po, master_full)
    p2, m2, v2, par = O.shard_step(po, want, mo, np.zeros_like(mo), np.zeros_like(mo), 1, ADAMW,
                                   wl["param_dtype"])
    assert_bitexact(to_host(md).reshape(R, po.S), p2, "master after accumulation")
    assert_bitexact(to_host(m).reshape(R, po.S), m2, "m after accumulation")
    assert_bitexact(to_host(v).reshape(R, po.S), v2, "v after accumulation")
    assert_bitexact(to_host(pd).reshape(R, po.S), par, "param after accumulation")


def test_accumulate_rejects_aliased_accumulators():
    pg = F.Plan([(16,)], 2, "flat")
    g = [torch.zeros(16, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    a = torch.zeros(16, device=DEV)
    with pytest.raises(F.FsdpError):
        F.fsdp_grad_accumulate(pg, g, [a, a], first=True)


# ----------------------------------------------------- DDP all-reduce
@pytest.mark.parametrize("R,gdt,odt", [(2, "f32", "f32"), (3, "bf16", "f32"), (8, "bf16", "bf16"),
                                       (5, "bf16", "f32"), (1, "f32", "bf16")])
def test_allreduce_avg_bit_exact(R, gdt, odt):
    banner(f"allreduce R={R} {gdt}->{odt}")
    rng = np.random.default_rng(R)
    shapes = [(37, 29), (1001,), (3, 5, 7)]
    pg = F.Plan(shapes, R, "per_param")
    T = pg.T
    grads = [(rng.standard_normal(T) * 1e-2).astype(np.float32) for _ in range(R)]
    if gdt == "bf16":
        grads = [O.bf16_rne(g) for g in grads]
    out = [torch.empty(T, dtype=torch.bfloat16 if odt == "bf16" else torch.float32, device=DEV)
           for _ in range(R)]
    F.fsdp_allreduce_avg(pg, [to_dev(g) for g in grads], out)
    want = O.allreduce_avg(grads)
    for r in range(R):
        w = O.bf16_rne(want[r]) if odt == "bf16" else want[r]
        assert_bitexact(to_host(out[r]), w, f"allreduce rank {r}")


@pytest.mark.parametrize("R,layout", [(2, "flat"), (3, "per_param"), (8, "per_param"),
                                      (13, "flat")])
def test_allreduce_is_reduce_scatter_then_gather(R, layout):
    """The all-reduce equals the reduce-scatter-average followed by the
    all-gather of the averaged fp32 shards ([FSDP2] 09), with the library's
    own calls on both sides: bit for bit."""
    rng = np.random.default_rng(100 + R)
    shapes = [(41, 7), (300,), (2, 3, 11)]
    pg = F.Plan(shapes, R, layout)
    T, S = pg.T, pg.S
    grads = [to_dev(O.bf16_rne((rng.standard_normal(T) * 1e-2).astype(np.float32)))
             for _ in range(R)]
    ar = [torch.empty(T, device=DEV) for _ in range(R)]
    F.fsdp_allreduce_avg(pg, grads, ar)
    rs = torch.empty(R * S, device=DEV)
    F.fsdp_reduce_scatter_avg(pg, grads, rs)
    full = [torch.empty(T, device=DEV) for _ in range(R)]
    F.fsdp_gather_unflatten(pg, rs, full)
    torch.cuda.synchronize()
    for r in range(R):
        assert torch.equal(ar[r].view(torch.int32), full[r].view(torch.int32)), r


def test_new_ops_reject_bad_arguments_before_launch():
    pg = F.Plan([(16, 4)], 2, "flat")
    other = F.Plan([(16, 4)], 4, "per_param")
    rs = F.Resharder(pg, other)
    buf = torch.zeros(2 * pg.S + 4 * other.S, device=DEV)
    src = buf[:2 * pg.S]
    with pytest.raises(F.FsdpError):        # source and destination overlap
        F.fsdp_reshard(rs, src, buf[1:1 + 4 * other.S])
    g = [torch.zeros(pg.T, device=DEV) for _ in range(2)]
    with pytest.raises(F.FsdpError):        # an output aliases a gradient
        F.fsdp_allreduce_avg(pg, g, [g[0], torch.zeros(pg.T, device=DEV)])
    o = torch.zeros(pg.T, device=DEV)
    with pytest.raises(F.FsdpError):        # two outputs are one buffer
        F.fsdp_allreduce_avg(pg, g, [o, o])
    with pytest.raises(ValueError):         # dtype mismatch, caught by the binding
        F.fsdp_reshard(rs, src, torch.zeros(4 * other.S, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert torch.count_nonzero(buf) == 0


def test_reshard_batch_moves_many_arrays_in_one_launch():
    shapes = shapes_of(BLOCK_512)
    pa, pb = O.plan_layout(shapes, 8, "per_param"), O.plan_layout(shapes, 3, "flat")
    rs = F.Resharder(F.Plan(shapes, 8, "per_param"), F.Plan(shapes, 3, "flat"))
    rng = np.random.default_rng(77)
    hs = [O.shard_pack(pa, rng.standard_normal(pa.T).astype(np.float32)) for _ in range(5)]
    srcs = [to_dev(h.reshape(-1)) for h in hs]
    dsts = [torch.full((3 * pb.S,), 5.0, device=DEV) for _ in hs]
    F.fsdp_reshard_batch(rs, srcs, dsts)
    for h, d in zip(hs, dsts):
        assert_bitexact(to_host(d).reshape(3, pb.S), O.reshard(pa, pb, h), "reshard batch")
    with pytest.raises(F.FsdpError):          # two destinations are one buffer
        F.fsdp_reshard_batch(rs, srcs[:2], [dsts[0], dsts[0]])
