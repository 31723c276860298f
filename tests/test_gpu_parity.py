"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: bit-exact for layout, pack, gather and reduce-scatter (fp32 sums in
rank order); AdamW master, m and v within max|d| <= 1e-6 * max(1, |ref|);
the bf16 recast within one bf16 ulp of the oracle's and exactly the RNE of
the GPU's own master.  Inputs come from the seeded generators in workloads/.
"""

import numpy as np
import pytest
import torch

import fully_sharded_amd as F
from oracle import fsdp_oracle as O
from tests.gpu_util import (assert_adamw_close, assert_bf16_within_ulp, assert_bitexact,
                            to_dev, to_host)
from workloads import gen
from workloads.configs import ADAMW, WORKLOADS, shapes_of

pytestmark = pytest.mark.gpu

SMALL = ["toy_2layer_r2", "block512_r4", "block512_flat_r4", "block512_r3", "block512_flat_r3"]
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    F.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def tdt(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def banner(msg):
    print(f"[gpu] {msg}", flush=True)


# ------------------------------------------------- full step, small workloads
@pytest.mark.parametrize("name", SMALL)
def test_step_parity_small_workloads(name):
    wl = WORKLOADS[name]
    R = wl["R"]
    banner(f"{name}: R={R} layout={wl['layout']}")
    for u, unit in enumerate(wl["units"]):
        shapes = shapes_of(unit)
        po = O.plan_layout(shapes, R, wl["layout"])
        pg = F.Plan(shapes, R, wl["layout"])
        assert (pg.T, pg.S) == (po.T, po.S)
        T, S = po.T, po.S
        master_full = gen.host_master(wl, u, shapes)
        full_d = to_dev(master_full)

        # a2: pack the fp32 master exactly and the parameter with its recast
        master_d = torch.empty(R * S, dtype=torch.float32, device=DEV)
        F.fsdp_shard_pack(pg, full_d, master_d)
        master_o = O.shard_pack(po, master_full)
        assert_bitexact(to_host(master_d).reshape(R, S), master_o, "pack fp32")
        pdt = wl["param_dtype"]
        param_d = torch.empty(R * S, dtype=tdt(pdt), device=DEV)
        F.fsdp_shard_pack(pg, full_d, param_d)
        param_o = O.bf16_rne(master_o) if pdt == "bf16" else master_o.copy()
        assert_bitexact(to_host(param_d).reshape(R, S), param_o, "pack+cast")
        m_d = torch.zeros(R * S, dtype=torch.float32, device=DEV)
        v_d = torch.zeros_like(m_d)
        m_o = np.zeros((R, S), np.float32)
        v_o = np.zeros((R, S), np.float32)

        for t in range(1, wl["steps"] + 1):
            # a3: all-gather + unflatten into R receivers
            recv = [torch.empty(T, dtype=tdt(pdt), device=DEV) for _ in range(R)]
            F.fsdp_gather_unflatten(pg, param_d, recv)
            full_o, views_o = O.gather_unflatten(po, param_o)
            for r in range(R):
                got = to_host(recv[r])
                if t == 1:
                    assert_bitexact(got, full_o, f"gather step {t} recv {r}")
                else:   # the parameters themselves may differ by an ulp here
                    if pdt == "bf16":
                        assert_bf16_within_ulp(got, full_o, "gather")
                    else:
                        assert_adamw_close(got, full_o, "gather")
            for p, view in enumerate(pg.unflatten(recv[0])):
                assert tuple(view.shape) == views_o[p].shape
            # gather of the GPU's own shards round-trips through pack exactly
            back = torch.empty_like(param_d)
            F.fsdp_shard_pack(pg, recv[R - 1], back)
            assert torch.equal(back.view(torch.int16) if pdt == "bf16" else back,
                               param_d.view(torch.int16) if pdt == "bf16" else param_d)

            grads = [gen.host_grad(wl, t, u, r, T) for r in range(R)]
            g_d = [to_dev(g) for g in grads]
            # a4: reduce-scatter-average
            rs_d = torch.empty(R * S, dtype=torch.float32, device=DEV)
            F.fsdp_reduce_scatter_avg(pg, g_d, rs_d)
            assert_bitexact(to_host(rs_d).reshape(R, S), O.reduce_scatter_avg(po, grads), "rs")

            # unfused AdamW on copies, for the fused/unfused identity below
            mc, mmc, vvc = master_d.clone(), m_d.clone(), v_d.clone()
            pc = torch.empty_like(param_d)
            F.fsdp_adamw_shard_step(pg, ADAMW, t, rs_d, mc, mmc, vvc, pc, grads_are_replicas=False)

            # a4+a5+a6 fused
            F.fsdp_adamw_shard_step(pg, ADAMW, t, g_d, master_d, m_d, v_d, param_d)
            master_o, m_o, v_o, param_o = O.shard_step(po, grads, master_o, m_o, v_o, t, ADAMW, pdt)
            gm = to_host(master_d).reshape(R, S)
            banner(f"{name} u={u} t={t}: master bit-exact fraction "
                   f"{np.mean(gm.view(np.uint32) == master_o.view(np.uint32)):.9f}")
            assert_adamw_close(gm, master_o, f"master t={t}")
            assert_adamw_close(to_host(m_d).reshape(R, S), m_o, f"m t={t}")
            assert_adamw_close(to_host(v_d).reshape(R, S), v_o, f"v t={t}")
            # stronger than the tolerance: the kernels evaluate the update in
            # IEEE double in the definition's order, as the oracle does, so
            # the rounded fp32 results agree bit for bit
            assert_bitexact(gm, master_o, f"master bits t={t}")
            assert_bitexact(to_host(m_d).reshape(R, S), m_o, f"m bits t={t}")
            assert_bitexact(to_host(v_d).reshape(R, S), v_o, f"v bits t={t}")
            gp = to_host(param_d).reshape(R, S)
            if pdt == "bf16":
                assert_bf16_within_ulp(gp, param_o, f"param t={t}")
                assert_bitexact(gp, O.bf16_rne(gm), "param is RNE of the GPU master")
            else:
                assert_adamw_close(gp, param_o, f"param t={t}")
                assert_bitexact(gp, gm, "fp32 param is the master")
            # fused == RS then AdamW, bit for bit
            assert_bitexact(to_host(mc), to_host(master_d), "fused vs unfused master")
            assert_bitexact(to_host(mmc), to_host(m_d), "fused vs unfused m")
            assert_bitexact(to_host(vvc), to_host(v_d), "fused vs unfused v")
            assert_bitexact(to_host(pc), to_host(param_d), "fused vs unfused param")
            # padding stays +0
            pad = O.shard_pack(po, np.ones(T, np.float32)) == 0
            for a in (gm, to_host(m_d).reshape(R, S), to_host(v_d).reshape(R, S)):
                assert np.all(a[pad].view(np.uint32) == 0)


# ------------------------------------------------ tiny ragged shapes, many R
def random_shapes(rng, R):
    shapes = []
    for _ in range(int(rng.integers(1, 6))):
        nd = int(rng.integers(1, 4))
        d0 = int(rng.integers(1, 3 * R + 3))
        shapes.append((d0,) + tuple(int(x) for x in rng.integers(1, 40, nd - 1)))
    return shapes


@pytest.mark.parametrize("R", [1, 2, 3, 5, 8, 13, 64])
def test_tiny_ragged_shapes_all_ops(R):
    rng = np.random.default_rng(1000 + R)
    banner(f"tiny ragged R={R}")
    for trial in range(12):
        shapes = random_shapes(rng, R)
        layout = O.FLAT if trial % 2 else O.PER_PARAM
        gdt = "bf16" if trial % 3 else "f32"
        pdt = "bf16" if trial % 4 != 1 else "f32"
        po = O.plan_layout(shapes, R, layout)
        pg = F.Plan(shapes, R, layout)
        assert (pg.T, pg.S) == (po.T, po.S)
        T, S = po.T, po.S
        master_full = rng.uniform(-1, 1, T).astype(np.float32)
        master_d = torch.empty(R * S, dtype=torch.float32, device=DEV)
        F.fsdp_shard_pack(pg, to_dev(master_full), master_d)
        master_o = O.shard_pack(po, master_full)
        assert_bitexact(to_host(master_d).reshape(R, S), master_o, "pack")
        p16 = O.bf16_rne(master_full)
        sh16 = torch.empty(R * S, dtype=torch.bfloat16, device=DEV)
        F.fsdp_shard_pack(pg, to_dev(p16), sh16)
        assert_bitexact(to_host(sh16).reshape(R, S), O.shard_pack(po, p16), "pack bf16")
        recv = [torch.empty(T, dtype=torch.bfloat16, device=DEV) if r % 3 != 2 else None
                for r in range(R)]
        F.fsdp_gather_unflatten(pg, sh16, recv)
        want, _ = O.gather_unflatten(po, O.shard_pack(po, p16))
        for r in range(R):
            if recv[r] is not None:
                assert_bitexact(to_host(recv[r]), want, "gather")
        grads = [(rng.standard_normal(T) * 1e-2).astype(np.float32) for _ in range(R)]
        if gdt == "bf16":
            grads = [O.bf16_rne(g) for g in grads]
        g_d = [to_dev(g) for g in grads]
        rs_d = torch.empty(R * S, dtype=torch.float32, device=DEV)
        F.fsdp_reduce_scatter_avg(pg, g_d, rs_d)
        assert_bitexact(to_host(rs_d).reshape(R, S), O.reduce_scatter_avg(po, grads), "rs")
        m_d = torch.zeros_like(master_d)
        v_d = torch.zeros_like(master_d)
        m_o = np.zeros((R, S), np.float32)
        v_o = np.zeros((R, S), np.float32)
        param_d = torch.empty(R * S, dtype=tdt(pdt), device=DEV)
        for t in (1, 2):
            F.fsdp_adamw_shard_step(pg, ADAMW, t, g_d, master_d, m_d, v_d, param_d)
            master_o, m_o, v_o, param_o = O.shard_step(po, grads, master_o, m_o, v_o, t, ADAMW, pdt)
            assert_adamw_close(to_host(master_d).reshape(R, S), master_o, "master")
            assert_adamw_close(to_host(m_d).reshape(R, S), m_o, "m")
            assert_adamw_close(to_host(v_d).reshape(R, S), v_o, "v")
            if pdt == "bf16":
                assert_bf16_within_ulp(to_host(param_d).reshape(R, S), param_o, "param")


def test_misaligned_base_pointers_take_the_scalar_path():
    """Views offset by a few elements (not 16-byte aligned) give the same bits."""
    banner("misaligned pointers")
    rng = np.random.default_rng(5)
    shapes = [(37, 11), (5,), (64, 8)]
    R = 3
    po = O.plan_layout(shapes, R, O.PER_PARAM)
    pg = F.Plan(shapes, R, O.PER_PARAM)
    T, S = po.T, po.S

    def off_view(n, dtype, k):
        base = torch.zeros(n + 16, dtype=dtype, device=DEV)
        return base[k:k + n]

    master_full = rng.uniform(-1, 1, T).astype(np.float32)
    full_d = off_view(T, torch.float32, 1)
    full_d.copy_(to_dev(master_full))
    master_d = off_view(R * S, torch.float32, 3)
    F.fsdp_shard_pack(pg, full_d, master_d)
    master_o = O.shard_pack(po, master_full)
    assert_bitexact(to_host(master_d).reshape(R, S), master_o, "pack misaligned")
    grads = [O.bf16_rne((rng.standard_normal(T) * 1e-3).astype(np.float32)) for _ in range(R)]
    g_d = []
    for q, g in enumerate(grads):
        x = off_view(T, torch.bfloat16, q + 1)
        x.copy_(to_dev(g))
        g_d.append(x)
    rs_d = off_view(R * S, torch.float32, 1)
    F.fsdp_reduce_scatter_avg(pg, g_d, rs_d)
    assert_bitexact(to_host(rs_d).reshape(R, S), O.reduce_scatter_avg(po, grads), "rs misaligned")
    m_d = off_view(R * S, torch.float32, 2)
    v_d = off_view(R * S, torch.float32, 1)
    p_d = off_view(R * S, torch.bfloat16, 5)
    F.fsdp_adamw_shard_step(pg, ADAMW, 1, g_d, master_d, m_d, v_d, p_d)
    mo, mm, vv, po16 = O.shard_step(po, grads, master_o, np.zeros((R, S), np.float32),
                                     np.zeros((R, S), np.float32), 1, ADAMW, "bf16")
    assert_adamw_close(to_host(master_d).reshape(R, S), mo, "master misaligned")
    assert_bf16_within_ulp(to_host(p_d).reshape(R, S), po16, "param misaligned")
    recv = [off_view(T, torch.bfloat16, r + 1) for r in range(R)]
    F.fsdp_gather_unflatten(pg, p_d, recv)
    want, _ = O.gather_unflatten(po, po16)
    back = off_view(R * S, torch.bfloat16, 7)
    F.fsdp_shard_pack(pg, recv[R - 1], back)
    assert torch.equal(back.view(torch.int16), p_d.view(torch.int16))
    for r in range(R):
        assert_bf16_within_ulp(to_host(recv[r]), want, "gather misaligned")


@pytest.mark.parametrize("R,aligned", [(8, True), (8, False), (9, True), (9, False)])
def test_short_reduce_scatter_and_adamw_two_element_forms(R, aligned):
    """The reduce-scatter alone and AdamW alone in short launches at R >= 8
    (two elements per lane: adjacent pairs on 16-byte aligned bases and even
    items, two strided elements otherwise; AdamW's odd-length tail element
    by element), on an odd-sized unit with bases aligned or a few elements
    off: bit for bit against the oracle, 2 steps."""
    shapes = [(75, 33), (7,), (40, 16), (9,)]
    po = O.plan_layout(shapes, R, O.PER_PARAM)
    pg = F.Plan(shapes, R, O.PER_PARAM)
    T, S = po.T, po.S
    assert (R * S) % 2 == (1 if R == 9 else 0)
    banner(f"short reduce-scatter + AdamW, R={R}, aligned={aligned}")
    rng = np.random.default_rng(400 + 2 * R + int(aligned))

    def place(a: np.ndarray, k: int):
        t = to_dev(a.reshape(-1))
        if aligned:
            return t
        base = torch.empty(t.numel() + 8, dtype=t.dtype, device=DEV)
        base[k:k + t.numel()].copy_(t)
        return base[k:k + t.numel()]

    master = O.shard_pack(po, rng.uniform(-1, 1, T).astype(np.float32))
    md, m_d, v_d = place(master, 1), place(np.zeros((R, S), np.float32), 3), \
        place(np.zeros((R, S), np.float32), 1)
    pd = place(np.zeros((R, S), np.uint16), 1)
    rs_d = place(np.zeros((R, S), np.float32), 3)
    mo, vo = np.zeros_like(master), np.zeros_like(master)
    for t in (1, 2):
        grads = [O.bf16_rne((rng.standard_normal(T) * 1e-2).astype(np.float32))
                 for _ in range(R)]
        F.fsdp_reduce_scatter_avg(pg, [place(g, 1 + q % 3) for q, g in enumerate(grads)], rs_d)
        rs = O.reduce_scatter_avg(po, grads)
        assert_bitexact(to_host(rs_d).reshape(R, S), rs, f"rs t={t}")
        F.fsdp_adamw_shard_step(pg, ADAMW, t, rs_d, md, m_d, v_d, pd, grads_are_replicas=False)
        master, mo, vo = O.adamw_step(master, mo, vo, rs, t, **ADAMW)
        assert_bitexact(to_host(md).reshape(R, S), master, f"master t={t}")
        assert_bitexact(to_host(m_d).reshape(R, S), mo, f"m t={t}")
        assert_bitexact(to_host(v_d).reshape(R, S), vo, f"v t={t}")
        assert_bitexact(to_host(pd).reshape(R, S), O.bf16_rne(master), f"param t={t}")


def test_nan_inf_and_signed_zero_propagate_like_the_oracle():
    banner("nan/inf")
    shapes = [(6, 4)]
    R = 2
    po = O.plan_layout(shapes, R, O.FLAT)
    pg = F.Plan(shapes, R, O.FLAT)
    T, S = po.T, po.S
    g0 = np.zeros(T, np.float32)
    g1 = np.zeros(T, np.float32)
    g0[0], g1[0] = -0.0, -0.0
    g0[1], g1[1] = -0.0, 0.0
    g0[2] = np.nan
    g0[3], g1[3] = np.inf, -np.inf
    g0[4], g1[4] = np.inf, 1.0
    g0[5], g1[5] = 3.4e38, 3.4e38
    grads = [g0, g1]
    g_d = [to_dev(g) for g in grads]
    rs_d = torch.empty(R * S, dtype=torch.float32, device=DEV)
    F.fsdp_reduce_scatter_avg(pg, g_d, rs_d)
    got = to_host(rs_d).reshape(R, S)
    with np.errstate(invalid="ignore", over="ignore"):   # inf - inf and overflow on purpose
        want = O.reduce_scatter_avg(po, grads)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert_bitexact(np.where(nan, 0, got), np.where(nan, 0, want), "rs specials")
    master = np.full((R, S), 0.5, np.float32)
    master_d = to_dev(master.reshape(-1))
    m_d = torch.zeros(R * S, device=DEV)
    v_d = torch.zeros(R * S, device=DEV)
    p_d = torch.empty(R * S, dtype=torch.bfloat16, device=DEV)
    F.fsdp_adamw_shard_step(pg, ADAMW, 1, g_d, master_d, m_d, v_d, p_d)
    with np.errstate(invalid="ignore", over="ignore"):
        mo, mm, vv, pp = O.shard_step(po, grads, master, np.zeros_like(master),
                                      np.zeros_like(master), 1, ADAMW, "bf16")
    assert_adamw_close(to_host(master_d).reshape(R, S), mo, "master specials")
    assert_bf16_within_ulp(to_host(p_d).reshape(R, S), pp, "param specials")


@pytest.mark.parametrize("R", [8, 16])
def test_specials_through_the_short_reduce_scatter_and_adamw(R):
    """NaN, +-Inf, -0 and overflow through the reduce-scatter alone and
    AdamW alone in short launches at R >= 8 (two elements per lane): in a
    rank's even piece (adjacent pairs) and in 1-element pieces (the strided
    path); the reduced gradient, master, m, v and the parameter equal the
    oracle's bit for bit, NaN compared by class."""
    shapes = [(2 * R, 6), (R // 2,)]
    po = O.plan_layout(shapes, R, O.PER_PARAM)
    pg = F.Plan(shapes, R, O.PER_PARAM)
    T, S = po.T, po.S
    banner(f"specials, short reduce-scatter + AdamW, R={R}")
    rng = np.random.default_rng(500 + R)
    grads = [(rng.standard_normal(T) * 1e-3).astype(np.float32) for _ in range(R)]
    for base in (0, 12 * R):       # the first parameter's and the second's first elements
        for g in grads:
            g[base] = -0.0
        grads[0][base + 1] = np.nan
        grads[1][base + 2], grads[2][base + 2] = np.inf, -np.inf
        grads[3][base + 3] = np.inf
    for g in grads:
        g[4] = 3.0e38
    grads = [O.bf16_rne(g) for g in grads]
    rs_d = torch.empty(R * S, dtype=torch.float32, device=DEV)
    F.fsdp_reduce_scatter_avg(pg, [to_dev(g) for g in grads], rs_d)
    with np.errstate(invalid="ignore", over="ignore"):
        rs = O.reduce_scatter_avg(po, grads)
    got = to_host(rs_d).reshape(R, S)
    nan = np.isnan(rs)
    assert nan.any() and np.isinf(rs).any()
    assert np.array_equal(np.isnan(got), nan)
    assert_bitexact(np.where(nan, 0, got), np.where(nan, 0, rs), "rs")
    master = O.shard_pack(po, rng.uniform(-1, 1, T).astype(np.float32))
    master[0, 0] = -0.0
    md = to_dev(master.reshape(-1))
    m_d, v_d = torch.zeros_like(md), torch.zeros_like(md)
    pd = torch.empty(R * S, dtype=torch.bfloat16, device=DEV)
    F.fsdp_adamw_shard_step(pg, ADAMW, 1, rs_d, md, m_d, v_d, pd, grads_are_replicas=False)
    with np.errstate(invalid="ignore", over="ignore"):
        mo, mm, vv = O.adamw_step(master, np.zeros_like(master), np.zeros_like(master), rs, 1,
                                  **ADAMW)
        pp = O.bf16_rne(mo)
    for got, want, name in ((to_host(md).reshape(R, S), mo, "master"),
                            (to_host(m_d).reshape(R, S), mm, "m"),
                            (to_host(v_d).reshape(R, S), vv, "v")):
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), name
        assert_bitexact(np.where(nan, 0, got), np.where(nan, 0, want), name)
    gq = to_host(pd).reshape(R, S)
    qnan = (pp & 0x7FFF) > 0x7F80
    assert np.array_equal((gq & 0x7FFF) > 0x7F80, qnan)
    assert_bitexact(np.where(qnan, 0, gq), np.where(qnan, 0, pp), "param")


def test_bf16_recast_over_every_fp32_pattern():
    """The kernels' fp32 -> bf16 rounding (the pack-cast kernel; the fused
    step stores its parameter through the same device function) on all
    2^32 fp32 bit patterns, in four launches of 2^30 elements: equal to
    torch's round-to-nearest-even GPU cast on every non-NaN input, NaN kept
    NaN; and equal to the oracle, bit for bit including NaN, on a window of
    2^20 patterns at the start and at the end of each launch (zeros,
    subnormals, the largest finite values, infinities and NaNs)."""
    n = 1 << 30
    pl = F.Plan([(n,)], 1, "flat")            # R = 1: the pack is the cast itself
    out = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    w = 1 << 20
    for c in range(4):
        banner(f"bf16 recast, fp32 patterns {c * n:#x}..{(c + 1) * n - 1:#x}")
        start = c * n if c * n < (1 << 31) else c * n - (1 << 32)   # as int32 bits
        bits_ = torch.arange(n, dtype=torch.int32, device=DEV).add_(start)
        x = bits_.view(torch.float32)
        F.fsdp_shard_pack(pl, x, out)
        ref = x.to(torch.bfloat16)
        nan = torch.isnan(x)
        diff = (out.view(torch.int16) != ref.view(torch.int16)) & ~nan
        assert int(diff.sum()) == 0, f"{int(diff.sum())} patterns differ from torch's cast"
        assert bool(torch.isnan(out.float())[nan].all()), "a NaN lost its class"
        for lo in (0, n - w):
            xs = to_host(x[lo:lo + w])
            assert_bitexact(to_host(out[lo:lo + w]), O.bf16_rne(xs), f"window {c}.{lo}")
        del bits_, x, ref, nan, diff
    torch.cuda.synchronize()


def test_repeat_runs_are_bit_identical():
    banner("determinism")
    wl = WORKLOADS["block512_r3"]
    shapes = shapes_of(wl["units"][0])
    pg = F.Plan(shapes, 3, "per_param")
    T, S = pg.T, pg.S
    grads = [gen.device_grad(wl, 1, 0, r, T, DEV) for r in range(3)]
    outs = []
    for _ in range(2):
        master = gen.device_master(wl, 0, shapes, DEV)
        md = torch.empty(3 * S, device=DEV)
        F.fsdp_shard_pack(pg, master, md)
        m = torch.zeros_like(md)
        v = torch.zeros_like(md)
        p = torch.empty(3 * S, dtype=torch.bfloat16, device=DEV)
        for t in (1, 2, 3):
            F.fsdp_adamw_shard_step(pg, ADAMW, t, grads, md, m, v, p)
        outs.append((md, m, v, p.view(torch.int16)))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_invalid_arguments_are_rejected_before_launch():
    banner("errors")
    pg = F.Plan([(8, 4)], 2, "flat")
    T, S = pg.T, pg.S
    buf = torch.zeros(4 * T, device=DEV)
    g = [buf[:T], buf[T:2 * T]]
    with pytest.raises(F.FsdpError) as e:     # output overlaps an input
        F.fsdp_reduce_scatter_avg(pg, g, buf[T // 2:T // 2 + 2 * S])
    assert e.value.status == -1
    master = torch.zeros(2 * S, device=DEV)
    m = torch.zeros(2 * S, device=DEV)
    p = torch.zeros(2 * S, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(F.FsdpError):          # step must be >= 1
        F.fsdp_adamw_shard_step(pg, ADAMW, 0, g, master, m, buf[2 * T:2 * T + 2 * S], p)
    with pytest.raises(F.FsdpError):          # eps must be > 0
        F.fsdp_adamw_shard_step(pg, dict(ADAMW, eps=0.0), 1, g, master, m,
                                buf[2 * T:2 * T + 2 * S], p)
    with pytest.raises(F.FsdpError):          # m aliases master
        F.fsdp_adamw_shard_step(pg, ADAMW, 1, g, master, master, buf[2 * T:2 * T + 2 * S], p)
    with pytest.raises(F.FsdpError):          # two receivers are the same buffer
        r = torch.zeros(T, dtype=torch.bfloat16, device=DEV)
        F.fsdp_gather_unflatten(pg, p, [r, r])
    torch.cuda.synchronize()
    assert torch.count_nonzero(master) == 0 and torch.count_nonzero(p.float()) == 0


# ------------------------------------------------------- full-size workloads
def sample_positions(rng, R, S, k):
    """Shard-space positions: random plus every rank's first/last element."""
    r = rng.integers(0, R, k)
    j = rng.integers(0, S, k)
    edge_r = np.repeat(np.arange(R), 2)
    edge_j = np.tile(np.array([0, S - 1]), R)
    return np.concatenate([r, edge_r]), np.concatenate([j, edge_j])


def flat_index(po, r, j):
    """Oracle layout: flat index of shard position (r, j), -1 for padding."""
    out = np.full(r.shape, -1, np.int64)
    for rr in range(po.R):
        sel = r == rr
        for f0, s0, n in po.pieces(rr):
            hit = sel & (j >= s0) & (j < s0 + n)
            out[hit] = f0 + (j[hit] - s0)
    return out


def test_model12_r8_full_step_bench_launch_configuration():
    """The 12-layer R=8 model, 3 steps, in the benchmark's default launch
    configuration: per step the gather of unit 0, then one launch per unit u
    holding u's fused step and unit u+1's gather (two alternating receive
    buffers), then unit 11's fused step alone.  Every unit's master, m, v
    and parameter are checked whole after every step, and every gather
    (every receiver of every unit, every step) against the oracle's gather
    of that unit's current parameter, all bit for bit."""
    wl = WORKLOADS["model12_r8"]
    R = wl["R"]
    shapes = shapes_of(wl["units"][0])
    po = O.plan_layout(shapes, R, wl["layout"])
    pg = F.Plan(shapes, R, wl["layout"])
    T, S = po.T, po.S
    n_units = len(wl["units"])
    last = n_units - 1
    banner(f"model12_r8: {n_units} units, T={T}, S={S}")
    state = []
    oracle = []
    for u in range(n_units):
        full = gen.device_master(wl, u, shapes, DEV)
        md = torch.empty(R * S, device=DEV)
        F.fsdp_shard_pack(pg, full, md)
        pd = torch.empty(R * S, dtype=torch.bfloat16, device=DEV)
        F.fsdp_shard_pack(pg, full, pd)
        state.append([md, torch.zeros_like(md), torch.zeros_like(md), pd])
        mo = O.shard_pack(po, to_host(full))
        oracle.append([mo, np.zeros_like(mo), np.zeros_like(mo), O.bf16_rne(mo)])
    recv = [[torch.empty(T, dtype=torch.bfloat16, device=DEV) for _ in range(R)]
            for _ in range(2)]

    def check_gather(u, t):
        """Every receiver of unit u's buffer holds the gather of u's
        current parameter (the oracle's, bit for bit)."""
        torch.cuda.synchronize()
        want, _ = O.gather_unflatten(po, oracle[u][3])
        for r in range(R):
            assert_bitexact(to_host(recv[u % 2][r]), want, f"gather u={u} t={t} recv {r}")

    for t in range(1, wl["steps"] + 1):
        F.fsdp_gather_unflatten(pg, state[0][3], recv[0])
        check_gather(0, t)
        for u in range(n_units):
            md, m, v, pd = state[u]
            grads = [gen.device_grad(wl, t, u, r, T, DEV) for r in range(R)]
            if u < last:
                F.fsdp_adamw_step_then_gather(pg, ADAMW, t, grads, md, m, v, pd, pg,
                                              state[u + 1][3], recv[(u + 1) % 2])
                check_gather(u + 1, t)
            else:
                F.fsdp_adamw_shard_step(pg, ADAMW, t, grads, md, m, v, pd)
            o = oracle[u]
            hg = [to_host(g) for g in grads]
            o[0], o[1], o[2], o[3] = O.shard_step(po, hg, o[0], o[1], o[2], t, ADAMW, "bf16")
            gm = to_host(md).reshape(R, S)
            assert_adamw_close(gm, o[0], f"master u={u} t={t}")
            assert_bitexact(gm, o[0], f"master bits u={u} t={t}")
            assert_bitexact(to_host(m).reshape(R, S), o[1], f"m u={u} t={t}")
            assert_bitexact(to_host(v).reshape(R, S), o[2], f"v u={u} t={t}")
            gp = to_host(pd).reshape(R, S)
            assert_bf16_within_ulp(gp, o[3], f"param u={u} t={t}")
            assert_bitexact(gp, o[3], f"param bits u={u} t={t}")
        banner(f"model12_r8 step {t} ok")


def test_group4096_flat_r8_one_step_whole():
    """One fused step of the 872,448,000-parameter group at R=8 (FSDP1
    FlatParameter), compared whole with the oracle run chunk by chunk on the
    host (1 Mi-element slices of the shard space on a thread pool: the
    oracle's rank-order mean, AdamW step and bf16 recast, element-wise), bit
    for bit on master, m, v and parameter.  The oracle's input is the
    FlatParameter's own definition: shard element j of rank r is element
    r*S + j of the full master."""
    from concurrent.futures import ThreadPoolExecutor
    wl = WORKLOADS["group4096_flat_r8"]
    R = wl["R"]
    shapes = shapes_of(wl["units"][0])
    po = O.plan_layout(shapes, R, wl["layout"])
    pg = F.Plan(shapes, R, wl["layout"])
    T, S = po.T, po.S
    assert R * S == T          # no padding at this size
    banner(f"group4096_flat_r8 whole step: T={T}")
    full = gen.device_master(wl, 0, shapes, DEV)
    md = torch.empty(R * S, device=DEV)
    F.fsdp_shard_pack(pg, full, md)
    pd = torch.empty(R * S, dtype=torch.bfloat16, device=DEV)
    F.fsdp_shard_pack(pg, full, pd)
    m = torch.zeros_like(md)
    v = torch.zeros_like(md)
    grads = [gen.device_grad(wl, 1, 0, r, T, DEV) for r in range(R)]
    F.fsdp_adamw_shard_step(pg, ADAMW, 1, grads, md, m, v, pd)
    torch.cuda.synchronize()
    chunk = 1 << 24
    sub = 1 << 20

    def oracle_slice(args):
        g, p0, a, b = args
        avg = O.rank_order_mean([x[a:b] for x in g])
        z = np.zeros(b - a, np.float32)
        p1, m1, v1 = O.adamw_step(p0[a:b], z, z, avg, 1, **ADAMW)
        return a, p1, m1, v1, O.bf16_rne(p1)

    with ThreadPoolExecutor(max_workers=8) as pool:
        for lo in range(0, T, chunk):
            hi = min(T, lo + chunk)
            g = [to_host(x[lo:hi]) for x in grads]
            p0 = to_host(full[lo:hi])
            want_p = np.empty(hi - lo, np.float32)
            want_m = np.empty_like(want_p)
            want_v = np.empty_like(want_p)
            want_q = np.empty(hi - lo, np.uint16)
            jobs = [(g, p0, a, min(hi - lo, a + sub)) for a in range(0, hi - lo, sub)]
            for a, p1, m1, v1, q1 in pool.map(oracle_slice, jobs):
                n = p1.size
                want_p[a:a + n], want_m[a:a + n], want_v[a:a + n], want_q[a:a + n] = \
                    p1, m1, v1, q1
            assert_bitexact(to_host(md[lo:hi]), want_p, f"master [{lo}, {hi})")
            assert_bitexact(to_host(m[lo:hi]), want_m, f"m [{lo}, {hi})")
            assert_bitexact(to_host(v[lo:hi]), want_v, f"v [{lo}, {hi})")
            assert_bitexact(to_host(pd[lo:hi]), want_q, f"param [{lo}, {hi})")
    banner("group4096 whole step ok")


def test_group4096_flat_r8_full_size_sampled():
    """The 4-block hidden-4096 group (872,448,000 parameters) as one FSDP1
    FlatParameter at R=8, at full size: pack, gather and 3 fused steps,
    checked on sampled elements against the oracle."""
    wl = WORKLOADS["group4096_flat_r8"]
    R = wl["R"]
    shapes = shapes_of(wl["units"][0])
    po = O.plan_layout(shapes, R, wl["layout"])
    pg = F.Plan(shapes, R, wl["layout"])
    T, S = po.T, po.S
    banner(f"group4096_flat_r8: T={T} S={S}")
    rng = np.random.default_rng(4096)
    rs_, js_ = sample_positions(rng, R, S, 65536)
    # also the parameter boundaries
    bnd = np.array([po.flat_off[p] + d for p in range(len(shapes)) for d in (0, -1) if
                    0 <= po.flat_off[p] + d < T])
    rs_ = np.concatenate([rs_, bnd // S])
    js_ = np.concatenate([js_, bnd % S])
    fi = flat_index(po, rs_, js_)
    assert np.all(fi >= 0)  # no padding at this size
    fi_d = torch.from_numpy(fi).to(DEV)
    idx = torch.from_numpy(rs_ * S + js_).to(DEV)

    full = gen.device_master(wl, 0, shapes, DEV)
    master_s = to_host(full[fi_d])
    md = torch.empty(R * S, device=DEV)
    F.fsdp_shard_pack(pg, full, md)
    pd = torch.empty(R * S, dtype=torch.bfloat16, device=DEV)
    F.fsdp_shard_pack(pg, full, pd)
    del full
    assert_bitexact(to_host(md[idx]), master_s, "pack sampled")
    assert_bitexact(to_host(pd[idx]), O.bf16_rne(master_s), "pack+cast sampled")
    recv = [torch.empty(T, dtype=torch.bfloat16, device=DEV) for _ in range(R)]
    F.fsdp_gather_unflatten(pg, pd, recv)
    for r in range(R):
        assert_bitexact(to_host(recv[r][fi_d]), O.bf16_rne(master_s), f"gather sampled {r}")
    for r in range(1, R):
        assert torch.equal(recv[0].view(torch.int16), recv[r].view(torch.int16))
    del recv
    torch.cuda.empty_cache()
    m = torch.zeros_like(md)
    v = torch.zeros_like(md)
    p0 = master_s
    m0 = np.zeros_like(p0)
    v0 = np.zeros_like(p0)
    for t in range(1, wl["steps"] + 1):
        grads = [gen.device_grad(wl, t, 0, r, T, DEV) for r in range(R)]
        F.fsdp_adamw_shard_step(pg, ADAMW, t, grads, md, m, v, pd)
        gs = [to_host(g[fi_d]) for g in grads]
        del grads
        p0, m0, v0 = O.adamw_step(p0, m0, v0, O.rank_order_mean(gs), t, **ADAMW)
        assert_adamw_close(to_host(md[idx]), p0, f"master t={t}")
        assert_adamw_close(to_host(m[idx]), m0, f"m t={t}")
        assert_adamw_close(to_host(v[idx]), v0, f"v t={t}")
        gp = to_host(pd[idx])
        assert_bf16_within_ulp(gp, O.bf16_rne(p0), f"param t={t}")
        assert_bitexact(gp, O.bf16_rne(to_host(md[idx])), "param = RNE(master)")
        banner(f"group4096 step {t} ok")


@pytest.mark.parametrize("R", [3, 8])
@pytest.mark.parametrize("layout", ["per_param", "flat"])
def test_wide_unit_gather_with_misaligned_ranks(layout, R):
    """A unit above 12.6M elements: at R=3 the gather's 8-byte-lane regime,
    at R=8 its 16-byte lanes with the 8 receivers' stores unrolled (units up
    to 40M elements).  Per parameter the shard length is odd, so every rank
    but 0 reads a misaligned source.  Gather and pack bit-exact, bf16 and
    fp32."""
    shapes = [(4099, 4099), (10,)]
    po = O.plan_layout(shapes, R, layout)
    pg = F.Plan(shapes, R, layout)
    assert 12582912 < po.T <= 41943040
    if layout == "per_param":
        assert po.S % 4 != 0      # ranks after 0 misaligned for 4-element lanes
    banner(f"wide gather {layout} R={R}: T={po.T} S={po.S}")
    rng = np.random.default_rng(99)
    for dt in ("bf16", "f32"):
        full = rng.standard_normal(po.T).astype(np.float32)
        if dt == "bf16":
            full = O.bf16_rne(full)
        sh = torch.empty(R * po.S, dtype=torch.bfloat16 if dt == "bf16" else torch.float32,
                         device=DEV)
        F.fsdp_shard_pack(pg, to_dev(full), sh)
        sh_o = O.shard_pack(po, full)
        assert_bitexact(to_host(sh).reshape(R, po.S), sh_o, f"pack {dt}")
        recv = [torch.empty(po.T, dtype=sh.dtype, device=DEV) for _ in range(R)]
        F.fsdp_gather_unflatten(pg, sh, recv)
        want, _ = O.gather_unflatten(po, sh_o)
        for r in range(R):
            assert_bitexact(to_host(recv[r]), want, f"gather {dt} receiver {r}")


def two_block_unit():
    from workloads.configs import BLOCK_512
    return shapes_of(BLOCK_512) + shapes_of(BLOCK_512)


def test_unfused_adamw_above_4096_workgroups_r8():
    """fsdp_adamw_shard_step with grads_are_replicas=0 (AdamW + recast on the
    reduce-scatter's fp32 output) on a two-block unit at R = 8: 6,146
    workgroups, the occupancy-capped launch; checked directly against the
    oracle's adamw_step of its reduce_scatter_avg, bit for bit, 2 steps."""
    shapes = two_block_unit()
    R = 8
    po = O.plan_layout(shapes, R, O.PER_PARAM)
    pg = F.Plan(shapes, R, O.PER_PARAM)
    T, S = po.T, po.S
    assert -(-R * S // 1024) > 4096
    banner(f"unfused AdamW R=8, {R * S} elements")
    rng = np.random.default_rng(77)
    master = O.shard_pack(po, rng.uniform(-0.05, 0.05, T).astype(np.float32))
    md = to_dev(master.reshape(-1))
    m_d = torch.zeros_like(md)
    v_d = torch.zeros_like(md)
    pd = torch.empty(R * S, dtype=torch.bfloat16, device=DEV)
    mo, vo = np.zeros_like(master), np.zeros_like(master)
    for t in (1, 2):
        grads = [O.bf16_rne((rng.standard_normal(T) * 1e-3).astype(np.float32))
                 for _ in range(R)]
        rs = O.reduce_scatter_avg(po, grads)
        F.fsdp_adamw_shard_step(pg, ADAMW, t, to_dev(rs.reshape(-1)), md, m_d, v_d, pd,
                                grads_are_replicas=False)
        master, mo, vo = O.adamw_step(master, mo, vo, rs, t, **ADAMW)
        assert_bitexact(to_host(md).reshape(R, S), master, f"master t={t}")
        assert_bitexact(to_host(m_d).reshape(R, S), mo, f"m t={t}")
        assert_bitexact(to_host(v_d).reshape(R, S), vo, f"v t={t}")
        assert_bitexact(to_host(pd).reshape(R, S), O.bf16_rne(master), f"param t={t}")


@pytest.mark.parametrize("gdt,pdt", [("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32"),
                                     ("f32", "f32")])
def test_fused_r8_above_4096_items_two_element_form(gdt, pdt):
    """The standalone fused step at R = 8 on a two-block unit (6,146 work
    items: the two-element kernel with its occupancy cap, where a one-block
    unit takes the one-element kernel), bit for bit against the oracle, 2
    steps, bf16 and fp32 gradients and parameters."""
    shapes = two_block_unit()
    R = 8
    po = O.plan_layout(shapes, R, O.PER_PARAM)
    pg = F.Plan(shapes, R, O.PER_PARAM)
    T, S = po.T, po.S
    assert len(pg.work_items(0)) > 4096
    banner(f"fused R=8 two-element form, {gdt} grads, {pdt} params")
    rng = np.random.default_rng(78)
    master = O.shard_pack(po, rng.uniform(-0.05, 0.05, T).astype(np.float32))
    md = to_dev(master.reshape(-1))
    m_d = torch.zeros_like(md)
    v_d = torch.zeros_like(md)
    pd = torch.empty(R * S, dtype=tdt(pdt), device=DEV)
    mo, vo = np.zeros_like(master), np.zeros_like(master)
    for t in (1, 2):
        grads = [(rng.standard_normal(T) * 1e-3).astype(np.float32) for _ in range(R)]
        if gdt == "bf16":
            grads = [O.bf16_rne(g) for g in grads]
        F.fsdp_adamw_shard_step(pg, ADAMW, t, [to_dev(g) for g in grads], md, m_d, v_d, pd)
        master, mo, vo, po16 = O.shard_step(po, grads, master, mo, vo, t, ADAMW, pdt)
        assert_bitexact(to_host(md).reshape(R, S), master, f"master t={t}")
        assert_bitexact(to_host(m_d).reshape(R, S), mo, f"m t={t}")
        assert_bitexact(to_host(v_d).reshape(R, S), vo, f"v t={t}")
        assert_bitexact(to_host(pd).reshape(R, S), po16, f"param t={t}")


def test_fused_r3_above_4096_items_misaligned_four_element_form():
    """The standalone fused step at R = 3 on a two-block per-parameter unit:
    6,147 work items, so the four-element kernel with its occupancy cap
    (short steps at R = 3 take the two-element kernel), whose ranks after 0
    read their gradient windows off the lane alignment (the funnelled
    loads).  Bit for bit against the oracle, 2 steps."""
    shapes = two_block_unit()
    R = 3
    po = O.plan_layout(shapes, R, O.PER_PARAM)
    pg = F.Plan(shapes, R, O.PER_PARAM)
    T, S = po.T, po.S
    items = pg.work_items(0)
    assert len(items) > 4096
    assert any((int(w[1]) - int(w[0])) % 4 != 0 for w in items if int(w[1]) >= 0)
    banner(f"fused R=3 four-element form, misaligned, {len(items)} items")
    rng = np.random.default_rng(79)
    master = O.shard_pack(po, rng.uniform(-0.05, 0.05, T).astype(np.float32))
    md = to_dev(master.reshape(-1))
    m_d = torch.zeros_like(md)
    v_d = torch.zeros_like(md)
    pd = torch.empty(R * S, dtype=torch.bfloat16, device=DEV)
    mo, vo = np.zeros_like(master), np.zeros_like(master)
    for t in (1, 2):
        grads = [O.bf16_rne((rng.standard_normal(T) * 1e-3).astype(np.float32))
                 for _ in range(R)]
        F.fsdp_adamw_shard_step(pg, ADAMW, t, [to_dev(g) for g in grads], md, m_d, v_d, pd)
        master, mo, vo, po16 = O.shard_step(po, grads, master, mo, vo, t, ADAMW, "bf16")
        assert_bitexact(to_host(md).reshape(R, S), master, f"master t={t}")
        assert_bitexact(to_host(m_d).reshape(R, S), mo, f"m t={t}")
        assert_bitexact(to_host(v_d).reshape(R, S), vo, f"v t={t}")
        assert_bitexact(to_host(pd).reshape(R, S), po16, f"param t={t}")


@pytest.mark.parametrize("R,shapes,aligned", [
    (8, [(2049, 2050), (9,)], True),     # even pieces, one 1-element piece
    (9, [(2043, 2049), (10,)], True),    # odd S: odd head and tail items
    (16, [(4100, 1030)], True),          # R > 8: the 64-slot instance
    (8, [(2049, 2050), (9,)], False),    # bases off 16-byte alignment
])
def test_long_fused_step_two_element_form(R, shapes, aligned):
    """The standalone fused step at R >= 8 with more than 4,096 work items:
    the two-element kernel (adjacent pairs where the item's offsets, length
    and the bases allow, else two strided elements), capped at 4 per CU.
    Bit for bit against the oracle (master, m, v, parameter), 2 steps."""
    po = O.plan_layout(shapes, R, O.PER_PARAM)
    pg = F.Plan(shapes, R, O.PER_PARAM)
    T, S = po.T, po.S
    items = pg.work_items(0)
    assert len(items) > 4096
    banner(f"fused two-element form, R={R}, {len(items)} items, aligned={aligned}")
    rng = np.random.default_rng(81 + R)

    def place(a: np.ndarray, k: int):
        """a on the device, k elements past a 256-byte aligned base."""
        t = to_dev(a)
        if aligned:
            return t
        base = torch.empty(t.numel() + 8, dtype=t.dtype, device=DEV)
        base[k:k + t.numel()].copy_(t)
        return base[k:k + t.numel()]

    master = O.shard_pack(po, rng.uniform(-0.05, 0.05, T).astype(np.float32))
    md = place(master.reshape(-1), 1)
    m_d = place(np.zeros(R * S, np.float32), 3)
    v_d = place(np.zeros(R * S, np.float32), 1)
    pd = place(np.zeros(R * S, np.uint16), 1)
    mo, vo = np.zeros_like(master), np.zeros_like(master)
    for t in (1, 2):
        grads = [O.bf16_rne((rng.standard_normal(T) * 1e-3).astype(np.float32))
                 for _ in range(R)]
        F.fsdp_adamw_shard_step(pg, ADAMW, t, [place(g, 1 + q % 5) for q, g in enumerate(grads)],
                                md, m_d, v_d, pd)
        master, mo, vo, po16 = O.shard_step(po, grads, master, mo, vo, t, ADAMW, "bf16")
        assert_bitexact(to_host(md).reshape(R, S), master, f"master t={t}")
        assert_bitexact(to_host(m_d).reshape(R, S), mo, f"m t={t}")
        assert_bitexact(to_host(v_d).reshape(R, S), vo, f"v t={t}")
        assert_bitexact(to_host(pd).reshape(R, S), po16, f"param t={t}")


@pytest.mark.parametrize("R", [3, 4, 8, 11])
def test_specials_through_the_short_fused_step(R):
    """NaN, +-Inf, -0 and overflow in the gradients of a short launch at
    R = 3 or 4 (the two-element kernel) or R >= 8 (the one-element kernel,
    specialised at 8, generic above):
    master, m, v and the parameter equal the oracle's bit for bit, NaN
    compared by class."""
    shapes = [(16, 5), (3,)]
    po = O.plan_layout(shapes, R, O.PER_PARAM)
    pg = F.Plan(shapes, R, O.PER_PARAM)
    T, S = po.T, po.S
    banner(f"specials, short fused step, R={R}")
    rng = np.random.default_rng(90 + R)
    grads = [(rng.standard_normal(T) * 1e-3).astype(np.float32) for _ in range(R)]
    for g in grads:
        g[0] = -0.0
    grads[0][1] = np.nan
    grads[1][2], grads[2][2] = np.inf, -np.inf
    grads[min(3, R - 1)][3] = np.inf
    for g in grads:
        g[4] = 3.0e38
    grads[0][5] = -0.0
    grads = [O.bf16_rne(g) for g in grads]
    master = O.shard_pack(po, rng.uniform(-1, 1, T).astype(np.float32))
    master[0, 0] = -0.0
    md = to_dev(master.reshape(-1))
    m_d = torch.zeros_like(md)
    v_d = torch.zeros_like(md)
    pd = torch.empty(R * S, dtype=torch.bfloat16, device=DEV)
    F.fsdp_adamw_shard_step(pg, ADAMW, 1, [to_dev(g) for g in grads], md, m_d, v_d, pd)
    with np.errstate(invalid="ignore", over="ignore"):
        mo, mm, vv, pp = O.shard_step(po, grads, master, np.zeros_like(master),
                                      np.zeros_like(master), 1, ADAMW, "bf16")
    for got, want, name in ((to_host(md).reshape(R, S), mo, "master"),
                            (to_host(m_d).reshape(R, S), mm, "m"),
                            (to_host(v_d).reshape(R, S), vv, "v")):
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), name
        assert_bitexact(np.where(nan, 0, got), np.where(nan, 0, want), name)
    gq = to_host(pd).reshape(R, S)
    qnan = (pp & 0x7FFF) > 0x7F80
    assert np.array_equal((gq & 0x7FFF) > 0x7F80, qnan)
    assert_bitexact(np.where(qnan, 0, gq), np.where(qnan, 0, pp), "param")


# AdamW hyper-parameters that give the kernels' divisions by the bias
# corrections 1 - b1^t and 1 - b2^t many different divisors: exact
# reciprocals (b = 1, powers of two), tiny ones (b near 2^-40) and generic
# ones, over steps from 1 to 123,457.
HP_SETS = [
    dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
    dict(lr=3e-4, beta1=0.95, beta2=0.98, eps=1e-6, weight_decay=0.1),
    dict(lr=1e-2, beta1=0.5, beta2=0.9, eps=1e-12, weight_decay=0.0),
    dict(lr=2e-3, beta1=0.0, beta2=0.0, eps=1e-8, weight_decay=0.05),
    dict(lr=1e-3, beta1=0.987654321, beta2=0.99987654321, eps=1e-8, weight_decay=0.01),
    dict(lr=1e-3, beta1=1 - 2.0**-20, beta2=1 - 2.0**-40, eps=1e-8, weight_decay=0.01),
]
HP_STEPS = (1, 2, 7, 1000, 123457)


def adamw_state(rng, po, T):
    """Master, m and v shards with nonzero moments, and R bf16 gradient
    replicas of which about 5% are exact zeros; the first 64 elements of
    the unit have zero gradient, m and v (m' = v' = 0)."""
    R = po.R
    master = O.shard_pack(po, rng.uniform(-1, 1, T).astype(np.float32))
    m = O.shard_pack(po, (rng.standard_normal(T) * 1e-3).astype(np.float32))
    v = O.shard_pack(po, np.abs(rng.standard_normal(T) * 1e-6).astype(np.float32))
    grads = []
    for _ in range(R):
        g = (rng.standard_normal(T) * 1e-3).astype(np.float32)
        g[rng.random(T) < 0.05] = 0.0
        g[:64] = 0.0
        grads.append(O.bf16_rne(g))
    for r in range(R):   # where rank r's shard holds the unit's first elements
        lo = r * po.S
        if lo < 64:
            n = min(64 - lo, po.S)
            m[r, :n] = 0.0
            v[r, :n] = 0.0
    return master, m, v, grads


def run_three_forms(hp, t, seed):
    """One step at step count t through the one-element fused kernel (R = 8,
    short launch), the four-element fused kernel (R = 5) and the unfused
    AdamW (R = 8, fp32 reduced gradient), each from its own random state,
    checked bit for bit against the oracle (master, m, v, parameter)."""
    shapes = [(512, 200), (777,)]
    for R, fused in ((8, True), (5, True), (8, False)):
        po = O.plan_layout(shapes, R, O.PER_PARAM)
        pg = F.Plan(shapes, R, O.PER_PARAM)
        T, S = po.T, po.S
        rng = np.random.default_rng(seed + 10 * R + int(fused))
        master, m, v, grads = adamw_state(rng, po, T)
        md, m_d, v_d = to_dev(master.reshape(-1)), to_dev(m.reshape(-1)), to_dev(v.reshape(-1))
        pd = torch.empty(R * S, dtype=torch.bfloat16, device=DEV)
        if fused:
            F.fsdp_adamw_shard_step(pg, hp, t, [to_dev(g) for g in grads], md, m_d, v_d, pd)
        else:
            rs = O.reduce_scatter_avg(po, grads)
            F.fsdp_adamw_shard_step(pg, hp, t, to_dev(rs.reshape(-1)), md, m_d, v_d, pd,
                                    grads_are_replicas=False)
        mo, mm, vv, pp = O.shard_step(po, grads, master, m, v, t, hp, "bf16")
        tag = f"R={R} {'fused' if fused else 'unfused'} t={t} b1={hp['beta1']} b2={hp['beta2']}"
        assert_bitexact(to_host(md).reshape(R, S), mo, "master " + tag)
        assert_bitexact(to_host(m_d).reshape(R, S), mm, "m " + tag)
        assert_bitexact(to_host(v_d).reshape(R, S), vv, "v " + tag)
        assert_bitexact(to_host(pd).reshape(R, S), pp, "param " + tag)


@pytest.mark.parametrize("k", range(len(HP_SETS)))
def test_adamw_bias_corrections_over_hparams_and_steps(k):
    """The division by each bias correction (a multiply and three fused
    multiply-adds with the host's two-part reciprocal) equals IEEE division:
    every kernel form bit for bit against the oracle over the step counts
    1, 2, 7, 1000 and 123,457."""
    hp = HP_SETS[k]
    banner(f"AdamW divisions, hparams {k}: {hp}")
    for t in HP_STEPS:
        run_three_forms(hp, t, 1000 * k + t)


def test_adamw_extreme_betas_take_the_ieee_division():
    """beta1 = beta2 = 2^-1000: where the gradient is zero, m' = b1 m and
    v' = b2 v fall below 2^-800 (v' into float64's subnormals), outside the
    fast division's range; those lanes branch to IEEE division, mixed in one
    wave with lanes that do not.  Bit for bit against the oracle."""
    hp = dict(lr=1e-3, beta1=2.0**-1000, beta2=2.0**-1000, eps=1e-8, weight_decay=0.01)
    banner("AdamW extreme betas")
    for t in (1, 3):
        run_three_forms(hp, t, 5000 + t)


@pytest.mark.parametrize("layout", [O.PER_PARAM, O.FLAT])
def test_sharded_step_equals_the_single_card_step(layout):
    """The equivalence check the FSDP2 page recommends (section 12: one card
    against the sharded ranks, the shards gathered back), on the GPU and
    through the library alone: R = 4 ranks stepping their shards on the R
    gradient replicas, then gathering master and parameter back to full
    tensors, equal bit for bit the R = 1 step on the rank-order mean of the
    replicas (the all-reduce's output), over 3 steps."""
    shapes = [(512, 96), (96, 130), (130,)]
    R = 4
    p4 = F.Plan(shapes, R, layout)
    p1 = F.Plan(shapes, 1, layout)
    T = p4.T
    banner(f"sharded vs single-card step, {layout}")
    rng = np.random.default_rng(123)
    full = torch.from_numpy(rng.uniform(-0.1, 0.1, T).astype(np.float32)).to(DEV)
    # R ranks: shards of master, m, v, parameter
    m4 = torch.empty(R * p4.S, device=DEV)
    F.fsdp_shard_pack(p4, full, m4)
    mm4, vv4 = torch.zeros_like(m4), torch.zeros_like(m4)
    pp4 = torch.empty(R * p4.S, dtype=torch.bfloat16, device=DEV)
    F.fsdp_shard_pack(p4, full, pp4)
    # one card: the full tensors
    m1 = full.clone()
    mm1, vv1 = torch.zeros_like(m1), torch.zeros_like(m1)
    pp1 = torch.empty(T, dtype=torch.bfloat16, device=DEV)
    F.fsdp_shard_pack(p1, full, pp1)
    for t in (1, 2, 3):
        grads = [to_dev(O.bf16_rne((rng.standard_normal(T) * 1e-3).astype(np.float32)))
                 for _ in range(R)]
        avg = [torch.empty(T, device=DEV) for _ in range(R)]
        F.fsdp_allreduce_avg(p4, grads, avg)
        F.fsdp_adamw_shard_step(p4, ADAMW, t, grads, m4, mm4, vv4, pp4)
        F.fsdp_adamw_shard_step(p1, ADAMW, t, avg[0], m1, mm1, vv1, pp1,
                                grads_are_replicas=False)
        for shards, one, dt in ((m4, m1, torch.float32), (mm4, mm1, torch.float32),
                                (vv4, vv1, torch.float32), (pp4, pp1, torch.bfloat16)):
            back = [torch.empty(T, dtype=dt, device=DEV)]
            F.fsdp_gather_unflatten(p4, shards, back + [None] * (R - 1))
            torch.cuda.synchronize()
            assert_bitexact(to_host(back[0]), to_host(one), f"{layout} t={t} {dt}")
