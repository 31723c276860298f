"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (fixtures under tests/golden, each citing its page and section),
closed forms, invariants, brute force on tiny inputs, exact rational
rounding, or a library routine (torch.optim.AdamW, torch's bf16 cast).
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fsdp_oracle as O
from workloads.configs import ADAMW, BLOCK_512, LINEARS_512, shapes_of

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def labels_to_values(labels, table):
    return np.array([table[x] for x in labels], np.float32)


# ------------------------------------------------------------ page examples
def test_walkthrough_toy_shards_gather_rs_and_comm():
    gd = golden("walkthrough_2rank_toy.json")
    R = gd["R"]
    # distinct, exactly representable values for the symbols
    w = {f"w{i}": np.float32(i * 1.5 - 2.0) for i in range(1, 9)}
    units = {}
    for name, labels in gd["units"].items():
        pl = O.plan_layout([(len(labels),)], R, O.PER_PARAM)
        full = labels_to_values(labels, w)
        sh = O.shard_pack(pl, full)
        units[name] = (pl, full, sh)
        for r in range(R):
            want = labels_to_values(gd["initial_shards"][str(r)][name], w)
            np.testing.assert_array_equal(sh[r], want)
        got, views = O.gather_unflatten(pl, sh)
        np.testing.assert_array_equal(got, labels_to_values(gd["all_gather_result"][name], w))
    # optimizer state covers exactly the rank's own elements (both units)
    for r in range(R):
        own = np.concatenate([units[n][2][r] for n in ("W1", "W2")])
        np.testing.assert_array_equal(own, labels_to_values(gd["optimizer_state_covers"][str(r)], w))

    # reduce-scatter-average of W2's gradients
    pl = units["W2"][0]
    g = {q: {f"g{i}": np.float32(0.25 * i + q * 3.0 - 1.0) for i in range(5, 9)} for q in range(R)}
    grads = [labels_to_values([f"g{i}" for i in range(5, 9)], g[q]) for q in range(R)]
    rs = O.reduce_scatter_avg(pl, grads)
    for r in range(R):
        want = np.array([(g[0][lab] + g[1][lab]) / 2 for lab in gd["reduce_scatter_avg_W2"][str(r)]],
                        np.float32)
        np.testing.assert_array_equal(rs[r], want)

    # one-step communication tally: 12 elements per rank vs 8 for DDP
    total = sum(O.comm_ledger(units[n][0], True)["total"] for n in ("W1", "W2"))
    assert total == gd["comm_per_rank_elements"]["fsdp_total"]
    assert total == sum(row[2] for row in gd["comm_per_rank_elements"]["rows"])
    per_op = O.comm_ledger(units["W1"][0], True)
    assert per_op["all_gather"] == 2 * 2 and per_op["reduce_scatter"] == 2 and per_op["optimizer"] == 0
    P = sum(len(v) for v in gd["units"].values())
    assert O.ddp_allreduce_elems(P, R) == gd["comm_per_rank_elements"]["ddp_allreduce"]


def test_fsdp2_eight_element_hand_calculation():
    gd = golden("fsdp2_8elem_hand_calc.json")
    R = gd["R"]
    w = {lab: np.float32(10 + 3 * i) for i, lab in enumerate(gd["w"])}
    full = labels_to_values(gd["w"], w)
    pl = O.plan_layout([(len(full),)], R, O.PER_PARAM)
    sh = O.shard_pack(pl, full)
    for r in range(R):
        np.testing.assert_array_equal(sh[r], labels_to_values(gd["resident"][str(r)], w))
    got, _ = O.gather_unflatten(pl, sh)
    np.testing.assert_array_equal(got, labels_to_values(gd["all_gather_result"], w))
    rng = np.random.default_rng(3)
    g = [rng.standard_normal(8).astype(np.float32) for _ in range(R)]
    rs = O.reduce_scatter_avg(pl, g)
    for r in range(R):
        lo, hi = gd["reduce_scatter_keeps"][str(r)]
        np.testing.assert_array_equal(rs[r], (g[0][lo:hi] + g[1][lo:hi]) / np.float32(2))


def test_fsdp2_exercise_sum_and_mean():
    gd = golden("fsdp2_exercise_rs.json")
    pl = O.plan_layout([(4,)], gd["R"], O.PER_PARAM)
    g = [np.array(gd["g0"], np.float32), np.array(gd["g1"], np.float32)]
    s = O.reduce_scatter_sum(pl, g)
    a = O.reduce_scatter_avg(pl, g)
    for r in range(2):
        np.testing.assert_array_equal(s[r], gd["sum_shards"][str(r)])
        np.testing.assert_array_equal(a[r], gd["mean_shards"][str(r)])
        np.testing.assert_array_equal(a[r], s[r] * np.float32(gd["mean_scale"]))


def test_block_layout_fsdp2_table_and_rows():
    gd = golden("block_layout_4gpu.json")
    R = gd["R"]
    names = [n for n, _ in BLOCK_512]
    shapes = shapes_of(BLOCK_512)
    for n, s in zip(names, shapes):
        assert list(s) == gd["params"][n]["shape"]
        assert int(np.prod(s)) == gd["params"][n]["numel"]
    pl = O.plan_layout(shapes, R, O.PER_PARAM)
    total_linears = 0
    for p, n in enumerate(names):
        info = gd["params"][n]
        if "per_gpu_shape" not in info:
            continue
        for r in range(R):
            f0, s0, cnt = O.Plan.pieces(pl, r)[p]
            assert cnt == info["per_gpu_numel"]
            assert [pl.k[p], pl.row[p]] == info["per_gpu_shape"]
        total_linears += info["per_gpu_numel"]
    assert total_linears == gd["fsdp2_per_gpu_total_linears"]
    assert abs(total_linears * 2 / 1e6 - gd["fsdp2_per_gpu_mb_fp16_approx"]) < 0.005
    # W_Q rows: GPU k holds rows 128k .. 128k+127
    full = np.zeros(pl.T, np.float32)
    q = pl.flat_off[0]
    full[q:q + 512 * 512] = np.repeat(np.arange(512, dtype=np.float32), 512)
    sh = O.shard_pack(pl, full)
    for r in range(R):
        lo, hi = gd["W_Q_rows_per_gpu"][str(r)]
        rows = sh[r, pl.shard_off[0]:pl.shard_off[0] + 128 * 512].reshape(128, 512)[:, 0]
        np.testing.assert_array_equal(rows, np.arange(lo, hi + 1))
    # block and 12-layer totals (the page rounds to 3.15M and 37.8M)
    assert round(pl.T / 1e6, 2) == gd["block_params_approx_millions"]
    assert round(gd["model_layers"] * pl.T / 1e6, 1) == gd["model_params_approx_millions"]
    lin = O.plan_layout(shapes_of(LINEARS_512), R, O.PER_PARAM)
    assert round(lin.T * 2 / 1e6, 1) == gd["block_mb_fp16_approx"]


def test_block_layout_flat_offsets_and_send_volume():
    gd = golden("block_layout_4gpu.json")
    R = gd["R"]
    assert [n for n, _ in LINEARS_512] == gd["flat_param_order"]
    pl = O.plan_layout(shapes_of(LINEARS_512), R, O.FLAT)
    assert pl.T == gd["flat_param_length"]
    offs = gd["flat_param_offsets"]
    for r in range(R):
        (f0, s0, n), = pl.pieces(r)
        assert (f0, f0 + n) == (offs[r], offs[r + 1]) and s0 == 0
    # the all-gather sends (N-1)/N of the layer: 3/4 * 6.3 MB ~ 4.7 MB (fp16)
    num, den = gd["all_gather_send_fraction"]
    sent_bytes = O.comm_ledger(pl, False)["all_gather"] * 2
    assert Fraction(sent_bytes, pl.T * 2) == Fraction(num, den)
    assert round(sent_bytes / 1e6, 1) == gd["all_gather_send_per_gpu_mb_fp16_approx"]


def test_memory_accounting_exercise_and_16_bytes():
    gd = golden("memory_accounting.json")
    ex = gd["exercise"]
    state = ex["weights_gb"] + ex["grads_gb"] + ex["optimizer_gb"]
    assert state / ex["R"] == ex["steady_per_card_gb"]
    assert O.peak_memory_lower_bound(state, ex["R"], ex["largest_group_gb"], ex["prefetch_gb"]) \
        == ex["peak_lower_bound_gb"]
    # 16 bytes per element: DDP holds 16P, a rank of R holds 16P/R (no padding at R=8)
    pl = O.plan_layout(shapes_of(BLOCK_512), 8, O.PER_PARAM)
    assert O.state_bytes_per_rank(pl) * 8 == gd["bytes_per_param_ddp"] * pl.T


# ------------------------------------------------------------- closed forms
def test_ceil_split_closed_forms_r3():
    pl = O.plan_layout(shapes_of(BLOCK_512), 3, O.PER_PARAM)
    rows = {p: [min(pl.k[p], max(0, pl.d0[p] - r * pl.k[p])) for r in range(3)]
            for p in range(len(pl.shapes))}
    assert rows[0] == [171, 171, 170]            # 512 rows
    assert rows[5] == [683, 683, 682]            # 2048 rows (W_down)
    assert pl.S == 1050454 and 3 * pl.S - pl.T == 4610
    assert [O.rank_valid(pl, r) for r in range(3)] == [pl.S, pl.S, pl.S - 4610]
    fl = O.plan_layout(shapes_of(BLOCK_512), 3, O.FLAT)
    assert fl.S == 1048918 and 3 * fl.S - fl.T == 2


def test_per_param_shard_sizes_match_row_counts():
    # d0 < R leaves later ranks empty; their pieces are pure padding
    pl = O.plan_layout([(2, 3), (5,)], 4, O.PER_PARAM)
    assert pl.k == [1, 2] and pl.S == 1 * 3 + 2
    assert [O.rank_valid(pl, r) for r in range(4)] == [3 + 2, 3 + 2, 0 + 1, 0]


# -------------------------------------------------------- brute force, tiny
def brute_owner(shapes, R, layout):
    """Per flat element: (rank, index in that rank's shard), found by walking
    the rows one by one (independent of the oracle's slicing)."""
    out = []
    if layout == O.FLAT:
        T = sum(int(np.prod(s)) for s in shapes)
        S = -(-T // R)
        return [(i // S, i % S) for i in range(T)], S
    base = 0
    for shape in shapes:
        d0 = shape[0]
        row = int(np.prod(shape)) // d0
        k = -(-d0 // R)
        for i in range(d0 * row):
            rr = i // row
            out.append((rr // k, base + (rr % k) * row + i % row))
        base += k * row
    return out, base


def random_shapes(rng, R):
    n = rng.integers(1, 5)
    shapes = []
    for _ in range(n):
        nd = rng.integers(1, 4)
        d0 = int(rng.integers(1, 2 * R + 2))
        shapes.append((d0,) + tuple(int(x) for x in rng.integers(1, 4, nd - 1)))
    return shapes


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("layout", [O.PER_PARAM, O.FLAT])
def test_brute_force_layout_pack_gather(R, layout):
    rng = np.random.default_rng(100 + R)
    for trial in range(25):
        shapes = random_shapes(rng, R)
        pl = O.plan_layout(shapes, R, layout)
        owner, S = brute_owner(shapes, R, layout)
        assert pl.S == S and pl.T == len(owner)
        full = rng.integers(1, 2**31, pl.T).astype(np.uint32)   # raw bit patterns
        sh = O.shard_pack(pl, full)
        want = np.zeros((R, S), np.uint32)
        for i, (r, j) in enumerate(owner):
            want[r, j] = full[i]
        np.testing.assert_array_equal(sh, want)
        back, views = O.gather_unflatten(pl, sh)
        np.testing.assert_array_equal(back, full)
        for p, v in enumerate(views):
            assert v.shape == pl.shapes[p]
        # invariants
        assert sum(O.rank_valid(pl, r) for r in range(R)) == pl.T
        if layout == O.FLAT:
            assert 0 <= R * pl.S - pl.T <= R - 1


@pytest.mark.parametrize("R", [1, 2, 3, 5, 8])
def test_brute_force_reduce_scatter(R):
    rng = np.random.default_rng(7 + R)
    for trial in range(10):
        shapes = random_shapes(rng, R)
        layout = O.PER_PARAM if trial % 2 else O.FLAT
        pl = O.plan_layout(shapes, R, layout)
        owner, S = brute_owner(shapes, R, layout)
        grads = [rng.standard_normal(pl.T).astype(np.float32) * np.float32(10.0 ** rng.integers(-3, 3))
                 for _ in range(R)]
        got = O.reduce_scatter_avg(pl, grads)
        want = np.zeros((R, S), np.float32)
        for i, (r, j) in enumerate(owner):
            acc = np.float32(grads[0][i])
            for q in range(1, R):
                acc = np.float32(acc + grads[q][i])
            want[r, j] = np.float32(acc / np.float32(R))
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def f32_round_exact(fr: Fraction) -> np.float32:
    """Round a rational to the nearest fp32 (ties to even), exactly."""
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    q, rem = divmod(a, ulp)
    q = int(q)
    if rem > ulp / 2 or (rem == ulp / 2 and q % 2 == 1):
        q += 1
    return np.float32(sign * float(q * ulp))


def test_reduce_scatter_division_correctly_rounded_r3():
    rng = np.random.default_rng(11)
    pl = O.plan_layout([(3, 7)], 3, O.FLAT)
    # integers up to 2^20: the fp32 sum of three is exact, so only the
    # division rounds, and it must round the exact quotient once
    grads = [rng.integers(-2**20, 2**20, pl.T).astype(np.float32) for _ in range(3)]
    out = O.reduce_scatter_avg(pl, grads)
    owner, _ = brute_owner([(3, 7)], 3, O.FLAT)
    for i, (r, j) in enumerate(owner):
        exact = Fraction(int(grads[0][i]) + int(grads[1][i]) + int(grads[2][i]), 3)
        assert out[r, j] == f32_round_exact(exact)


def test_reduce_scatter_is_slice_of_allreduce_and_identity_at_r1():
    rng = np.random.default_rng(5)
    shapes = shapes_of(BLOCK_512)[:3] + [(37, 5), (3,)]
    for R in (1, 3, 4):
        pl = O.plan_layout(shapes, R, O.PER_PARAM)
        g16 = [rng.integers(0, 2**16, pl.T).astype(np.uint16) & np.uint16(0x3FFF) for _ in range(R)]
        rs = O.reduce_scatter_avg(pl, g16)
        # all-reduce-average of the whole vector, written directly, then sliced
        total = O.bf16_to_f32(g16[0]).copy()
        for q in range(1, R):
            total = total + O.bf16_to_f32(g16[q])
        mean = total / np.float32(R)
        np.testing.assert_array_equal(rs, O.shard_pack(pl, mean))
        if R == 1:
            np.testing.assert_array_equal(rs[0][:pl.T], O.bf16_to_f32(g16[0]))


def test_reduce_scatter_signed_zero_and_nan():
    pl = O.plan_layout([(4,)], 2, O.FLAT)
    z = np.float32(-0.0)
    g0 = np.array([z, z, np.nan, np.inf], np.float32)
    g1 = np.array([z, 0.0, 1.0, -np.inf], np.float32)
    with np.errstate(invalid="ignore"):                # inf - inf is the point
        out = O.reduce_scatter_avg(pl, [g0, g1]).reshape(-1)
    assert np.signbit(out[0]) and out[0] == 0          # -0 + -0 stays -0
    assert not np.signbit(out[1]) and out[1] == 0      # -0 + +0 is +0
    assert np.isnan(out[2]) and np.isnan(out[3])       # NaN, inf - inf


# ---------------------------------------------------------------------- AdamW
def torch_adamw_one_step(p, m, v, g, t):
    """torch.optim.AdamW in float64, from the given state, one step."""
    pt = torch.tensor(p, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([pt], lr=ADAMW["lr"], betas=(ADAMW["beta1"], ADAMW["beta2"]),
                            eps=ADAMW["eps"], weight_decay=ADAMW["weight_decay"], foreach=False)
    opt.state[pt] = {"step": torch.tensor(float(t - 1), dtype=torch.float64),
                     "exp_avg": torch.tensor(m, dtype=torch.float64),
                     "exp_avg_sq": torch.tensor(v, dtype=torch.float64)}
    pt.grad = torch.tensor(g, dtype=torch.float64)
    opt.step()
    st = opt.state[pt]
    return pt.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def ulp32(x):
    return np.spacing(np.abs(np.asarray(x, np.float32)))


@pytest.mark.parametrize("t", [1, 2, 3, 10, 1000])
def test_adamw_matches_torch_adamw_float64(t):
    rng = np.random.default_rng(t)
    n = 20000
    p = rng.uniform(-0.05, 0.05, n).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32) if t > 1 else np.zeros(n, np.float32)
    v = (rng.uniform(0, 1, n) * 1e-6).astype(np.float32) if t > 1 else np.zeros(n, np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    p2, m2, v2 = O.adamw_step(p, m, v, g, t, **ADAMW)
    tp, tm, tv = torch_adamw_one_step(p, m, v, g, t)
    for ours, ref in ((p2, tp), (m2, tm), (v2, tv)):
        # torch's float64 result and ours agree to within one fp32 ulp.  Exact
        # fp32 ties are common here ((9m + g)/10 of two fp32 values often sits
        # on a midpoint), and there the float64 rounding of 0.9 and torch's
        # lerp form decide the side, so equality is not required everywhere.
        assert np.all(np.abs(ours.astype(np.float64) - ref) <= ulp32(ref))
        assert np.mean(ours == ref.astype(np.float32)) > 0.99


def test_adamw_closed_form_first_step_and_zero_grad():
    rng = np.random.default_rng(1)
    n = 5000
    p = rng.uniform(-1, 1, n).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    g[:10] = 0.0
    zero = np.zeros(n, np.float32)
    lr, wd, eps = ADAMW["lr"], ADAMW["weight_decay"], ADAMW["eps"]
    p2, m2, v2 = O.adamw_step(p, zero, zero, g, 1, **ADAMW)
    # t=1 from zero moments: m_hat = g and v_hat = g^2 exactly
    g64 = g.astype(np.float64)
    want = p.astype(np.float64) * (1 - lr * wd) - lr * g64 / (np.abs(g64) + eps)
    assert np.all(np.abs(p2 - want) <= ulp32(want))
    # g = 0: pure decay, moments stay zero
    np.testing.assert_array_equal(p2[:10], (p[:10].astype(np.float64) * (1 - lr * wd)).astype(np.float32))
    assert np.all(m2[:10] == 0) and np.all(v2[:10] == 0)


def test_shard_step_equals_full_step_sliced_and_padding_stays_zero():
    rng = np.random.default_rng(9)
    shapes = [(5, 3), (7,), (2, 2, 2)]
    R = 3
    pl = O.plan_layout(shapes, R, O.PER_PARAM)
    full_master = rng.uniform(-1, 1, pl.T).astype(np.float32)
    master = O.shard_pack(pl, full_master)
    m = np.zeros_like(master)
    v = np.zeros_like(master)
    fm = full_master.copy()
    fmm = np.zeros(pl.T, np.float32)
    fvv = np.zeros(pl.T, np.float32)
    pad = O.shard_pack(pl, np.ones(pl.T, np.float32)) == 0
    assert pad.any()
    for t in (1, 2, 3):
        grads = [rng.standard_normal(pl.T).astype(np.float32) for _ in range(R)]
        master, m, v, param = O.shard_step(pl, grads, master, m, v, t, ADAMW, "bf16")
        # one device holding everything, stepping on the mean gradient
        mean = grads[0].copy()
        for q in range(1, R):
            mean = mean + grads[q]
        mean = mean / np.float32(R)
        fm, fmm, fvv = O.adamw_step(fm, fmm, fvv, mean, t, **ADAMW)
        np.testing.assert_array_equal(master, O.shard_pack(pl, fm))
        np.testing.assert_array_equal(m, O.shard_pack(pl, fmm))
        np.testing.assert_array_equal(v, O.shard_pack(pl, fvv))
        np.testing.assert_array_equal(param, O.bf16_rne(master))
        for a in (master, m, v):
            assert np.all(a[pad].view(np.uint32) == 0)
        back, _ = O.gather_unflatten(pl, param)
        np.testing.assert_array_equal(back, O.bf16_rne(fm))


# ---------------------------------------------------------------------- bf16
def bf16_exact(x: np.float32) -> int:
    """Nearest bf16 (ties to even) by exact rational arithmetic."""
    if np.isnan(x):
        return -1
    if np.isinf(x):
        return 0x7F80 if x > 0 else 0xFF80
    fr = Fraction(float(x))
    sign = 0x8000 if (fr < 0 or (fr == 0 and np.signbit(x))) else 0
    a = abs(fr)
    best = None
    # candidates: the two bf16 values around a (scan by exponent)
    cands = []
    u = int(np.float32(float(a)).view(np.uint32)) >> 16
    for h in (u - 1, u, u + 1, u + 2):
        if 0 <= h <= 0x7F80:
            val = Fraction(float(np.uint32(h << 16).view(np.float32))) if h < 0x7F80 else None
            cands.append((h, val))
    max_bf16 = Fraction(float(np.uint32(0x7F7F << 16).view(np.float32)))
    half_ulp_top = Fraction(2) ** (127 - 8)   # half of the bf16 ulp at the top binade
    if a >= max_bf16 + half_ulp_top:
        return sign | 0x7F80
    for h, val in cands:
        if val is None:
            continue
        d = abs(val - a)
        if best is None or d < best[0] or (d == best[0] and h % 2 == 0):
            best = (d, h)
    return sign | best[1]


def test_bf16_rne_exact_rational_on_edge_cases():
    vals = [0.0, -0.0, 1.0, -1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, 1 - 2**-9,
            3.0e38, 3.3895313e38, 3.39e38, -3.39e38, 1e-38, 1e-40, -1e-45, 2**-133, 2**-134,
            65504.0, 0.1, 1.0 / 3.0, np.inf, -np.inf]
    x = np.array(vals, np.float32)
    got = O.bf16_rne(x)
    for xi, gi in zip(x, got):
        assert int(gi) == bf16_exact(xi), (xi, hex(gi))


def test_bf16_rne_random_patterns_vs_exact_and_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    got = O.bf16_rne(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)
    for xi in x[:300]:
        assert int(O.bf16_rne(np.array([xi]))[0]) == bf16_exact(xi)
    # exact ties: low half exactly 0x8000, both parities
    tie = (rng.integers(0, 0x7F00, 2000).astype(np.uint32) << 16) | np.uint32(0x8000)
    t = O.bf16_rne(tie.view(np.float32))
    hi = tie >> 16
    np.testing.assert_array_equal(t, np.where(hi % 2 == 1, hi + 1, hi).astype(np.uint16))


def test_bf16_nan_stays_nan():
    x = np.array([np.nan, -np.nan], np.float32)
    x = np.concatenate([x, np.array([0x7F800001, 0xFFC00000, 0x7FFFFFFF], np.uint32).view(np.float32)])
    r = O.bf16_rne(x)
    back = O.bf16_to_f32(r)
    assert np.all(np.isnan(back))


def test_bf16_to_f32_over_every_bf16_pattern():
    """The oracle's bf16 -> fp32 widening on all 65,536 bf16 bit patterns:
    equal, bit for bit (NaN payloads included), to torch's bfloat16 -> float32
    conversion (a library routine), and to the value the bf16 fields define
    on the normal, subnormal, zero and infinite classes:
    (-1)^s * 2^(e - 127) * (1 + f/128), or 2^-126 * f/128 when e = 0."""
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_to_f32(u)
    ref = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))
    s = (u >> 15).astype(np.int64)
    e = ((u >> 7) & 0xFF).astype(np.int64)
    f = (u & 0x7F).astype(np.int64)
    fin = e < 0xFF
    mag = np.where(e > 0, np.ldexp(1.0 + f / 128.0, (e - 127).clip(-126, 127)),
                   np.ldexp(f / 128.0, -126))
    want = np.where(s == 1, -mag, mag)
    np.testing.assert_array_equal(ours[fin].astype(np.float64), want[fin])
    assert np.all(np.signbit(ours) == (s == 1))
    inf = (e == 0xFF) & (f == 0)
    assert np.all(np.isinf(ours[inf])) and np.all(np.isnan(ours[(e == 0xFF) & (f != 0)]))
    assert ours[0x3F80] == 1.0 and ours[0xC000] == -2.0 and ours[0x0001] == 2.0 ** -133


def test_bf16_rne_over_every_fp32_pattern_matches_torch():
    """All 2^32 fp32 bit patterns, in 64 chunks on 8 threads (about 20 s):
    the oracle's recast equals torch's round-to-nearest-even cast (a library
    routine) on every non-NaN input, and keeps every NaN a NaN (torch
    returns one canonical NaN, so only the class is compared)."""
    from concurrent.futures import ThreadPoolExecutor

    chunk = 1 << 26

    def check(c):
        x = (np.arange(chunk, dtype=np.uint32) + np.uint32(c * chunk)).view(np.float32)
        ours = O.bf16_rne(x)
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(x)
        return (int(np.count_nonzero(ours[~nan] != ref[~nan])),
                int(np.count_nonzero((ours[nan] & 0x7FFF) <= 0x7F80)))

    threads = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with ThreadPoolExecutor(8) as ex:
            bad = list(ex.map(check, range((1 << 32) // chunk)))
    finally:
        torch.set_num_threads(threads)
    assert all(b == (0, 0) for b in bad), [(i, b) for i, b in enumerate(bad) if b != (0, 0)]


# ---------------------------------------------------------------- isolation
def test_oracle_is_independent_of_the_library():
    here = os.path.dirname(O.__file__)
    for fn in os.listdir(here):
        if fn.endswith(".py"):
            with open(os.path.join(here, fn)) as f:
                src = f.read()
            assert "fully_sharded_amd" not in src and "ctypes" not in src


# ------------------------------------------------------------ next rows
def test_reshard_block_r4_to_r2_matches_the_page_row_table():
    """[BLOCK] 4-GPU table: W_Q rows 128k..128k+127 on GPU k.  At 2 ranks
    rank 0 must hold rows 0..255, i.e. what GPUs 0 and 1 held, in order."""
    shapes = shapes_of(BLOCK_512)
    p4 = O.plan_layout(shapes, 4, O.PER_PARAM)
    p2 = O.plan_layout(shapes, 2, O.PER_PARAM)
    full = np.zeros(p4.T, np.float32)
    full[:512 * 512] = np.repeat(np.arange(512, dtype=np.float32), 512)
    s2 = O.reshard(p4, p2, O.shard_pack(p4, full))
    rows0 = s2[0, :256 * 512].reshape(256, 512)[:, 0]
    rows1 = s2[1, :256 * 512].reshape(256, 512)[:, 0]
    np.testing.assert_array_equal(rows0, np.arange(256))
    np.testing.assert_array_equal(rows1, np.arange(256, 512))


@pytest.mark.parametrize("Ra,Rb", [(1, 3), (2, 8), (3, 2), (5, 4), (8, 8)])
def test_reshard_brute_force_roundtrip_and_layout_change(Ra, Rb):
    rng = np.random.default_rng(Ra * 10 + Rb)
    for trial in range(12):
        shapes = random_shapes(rng, max(Ra, Rb))
        la = O.FLAT if trial % 2 else O.PER_PARAM
        lb = O.PER_PARAM if trial % 3 else O.FLAT
        pa = O.plan_layout(shapes, Ra, la)
        pb = O.plan_layout(shapes, Rb, lb)
        x = rng.integers(1, 2**31, pa.T).astype(np.uint32)
        sa = O.shard_pack(pa, x)
        sb = O.reshard(pa, pb, sa)
        # brute force: each destination element found through the two owner maps
        own_a, _ = brute_owner(shapes, Ra, la)
        own_b, Sb = brute_owner(shapes, Rb, lb)
        want = np.zeros((Rb, Sb), np.uint32)
        for i in range(pa.T):
            ra, ja = own_a[i]
            rb, jb = own_b[i]
            want[rb, jb] = sa[ra, ja]
        np.testing.assert_array_equal(sb, want)
        np.testing.assert_array_equal(O.reshard(pb, pa, sb), sa)      # round trip
        np.testing.assert_array_equal(O.reshard(pa, pa, sa), sa)      # identity


def test_grad_accumulate_order_and_single_micro_batch():
    rng = np.random.default_rng(2)
    g = [(rng.standard_normal(1000) * 10.0 ** rng.integers(-6, 3)).astype(np.float32)
         for _ in range(5)]
    acc = O.grad_accumulate(g)
    want = g[0].copy()
    for k in range(1, 5):
        for i in range(1000):
            want[i] = np.float32(want[i] + g[k][i])
    np.testing.assert_array_equal(acc.view(np.uint32), want.view(np.uint32))
    np.testing.assert_array_equal(O.grad_accumulate([g[0]]), g[0])
    # integers below 2^20: the fp32 sum is exact
    ints = [rng.integers(-2**20, 2**20, 64).astype(np.float32) for _ in range(7)]
    np.testing.assert_array_equal(O.grad_accumulate(ints),
                                  np.sum(np.stack(ints).astype(np.int64), 0).astype(np.float32))
    z = np.array([-0.0], np.float32)
    assert np.signbit(O.grad_accumulate([z, z])[0])
    b16 = [O.bf16_rne(x) for x in g[:2]]
    np.testing.assert_array_equal(O.grad_accumulate(b16),
                                  O.bf16_to_f32(b16[0]) + O.bf16_to_f32(b16[1]))


def test_allreduce_is_gather_of_reduce_scatter_and_ddp_volume():
    rng = np.random.default_rng(4)
    shapes = [(7, 3), (10,), (3, 2, 2)]
    for R in (1, 2, 3, 8):
        for layout in (O.PER_PARAM, O.FLAT):
            pl = O.plan_layout(shapes, R, layout)
            g = [rng.standard_normal(pl.T).astype(np.float32) for _ in range(R)]
            ar = O.allreduce_avg(g)
            gathered, _ = O.gather_unflatten(pl, O.reduce_scatter_avg(pl, g))
            for r in range(R):
                np.testing.assert_array_equal(ar[r], gathered)
    # the walkthrough's DDP comparison: 2(N-1)/N x 8 = 8 elements at N = 2
    gd = golden("walkthrough_2rank_toy.json")
    assert O.ddp_allreduce_elems(8, 2) == gd["comm_per_rank_elements"]["ddp_allreduce"]
