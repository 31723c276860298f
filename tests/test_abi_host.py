"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every function include/fsdp_mi355x.h declares, and its shapes-only plan agrees
with the oracle's independently written layout."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import fully_sharded_amd as F
from oracle import fsdp_oracle as O
from workloads.configs import WORKLOADS, shapes_of

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fsdp_mi355x.h")


def declared_functions():
    with open(HEADER) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fsdp_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert "fsdp_plan_layout" in names and "fsdp_adamw_shard_step" in names
    L = ctypes.CDLL(F.binding.LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"{n} declared but not exported"
    for n in ("fsdp_plan_layout", "fsdp_shard_pack", "fsdp_gather_unflatten",
              "fsdp_reduce_scatter_avg", "fsdp_adamw_shard_step"):
        assert n in names


def test_status_strings():
    L = F.lib()
    assert L.fsdp_status_string(0) == b"ok"
    assert L.fsdp_status_string(-1) == b"invalid argument"


def check_plan(shapes, R, layout):
    po = O.plan_layout(shapes, R, layout)
    pg = F.Plan(shapes, R, layout)
    assert (pg.T, pg.S, pg.R, pg.n_params) == (po.T, po.S, R, len(shapes))
    for p in range(len(shapes)):
        q = pg.param(p)
        assert q["flat_off"] == po.flat_off[p] and q["numel"] == po.numel[p]
        assert q["rows_per_shard"] == po.k[p] and q["row_numel"] == po.row[p]
        if layout == O.PER_PARAM:
            assert q["shard_off"] == po.shard_off[p]
    for r in range(R):
        assert pg.rank_valid(r) == O.rank_valid(po, r)
    # the segments are exactly the oracle's pieces (merged where contiguous)
    seg = pg.segments()
    merged = []
    for r in range(R):
        for f0, s0, n in po.pieces(r):
            if n == 0:
                continue
            if merged and merged[-1][0] == r and merged[-1][1] + merged[-1][3] == s0 \
                    and merged[-1][2] + merged[-1][3] == f0:
                merged[-1] = (r, merged[-1][1], merged[-1][2], merged[-1][3] + n)
            else:
                merged.append((r, s0, f0, n))
    assert seg == merged
    for raf in (True, False):
        assert pg.comm_ledger(raf) == O.comm_ledger(po, raf)
    assert pg.state_bytes_per_rank() == O.state_bytes_per_rank(po)
    if R * po.S > 1 << 22:
        return
    # and, expanded to elements, the same map as the oracle's
    got = np.full((R, po.S), -1, np.int64)
    for rank, s0, f0, n in seg:
        assert n > 0 and 0 <= s0 and s0 + n <= po.S
        got[rank, s0:s0 + n] = np.arange(f0, f0 + n)
    want = np.full((R, po.S), -1, np.int64)
    for r in range(R):
        for f0, s0, n in po.pieces(r):
            want[r, s0:s0 + n] = np.arange(f0, f0 + n)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_plan_matches_oracle_on_workloads(name):
    wl = WORKLOADS[name]
    check_plan(shapes_of(wl["units"][0]), wl["R"], wl["layout"])


@pytest.mark.parametrize("R", [1, 2, 3, 4, 7, 8, 16, 64])
def test_plan_matches_oracle_on_random_tiny_shapes(R):
    rng = np.random.default_rng(R)
    for trial in range(30):
        shapes = []
        for _ in range(int(rng.integers(1, 6))):
            nd = int(rng.integers(1, 4))
            shapes.append((int(rng.integers(1, 2 * R + 2)),) +
                          tuple(int(x) for x in rng.integers(1, 5, nd - 1)))
        check_plan(shapes, R, O.PER_PARAM if trial % 2 else O.FLAT)


def test_plan_rejects_bad_arguments():
    L = F.lib()

    def plan(shapes, R, layout, ndims=None):
        nd = ndims if ndims is not None else [len(s) for s in shapes]
        flat = [d for s in shapes for d in s] or [0]
        h = ctypes.c_void_p(1234)
        st = L.fsdp_plan_layout(len(nd), (ctypes.c_int32 * max(1, len(nd)))(*nd),
                                (ctypes.c_int64 * len(flat))(*flat), R, layout, ctypes.byref(h))
        if st == 0:
            L.fsdp_plan_destroy(h)
        else:
            assert h.value is None
        return st

    assert plan([(4,)], 2, 0) == 0
    assert plan([], 2, 0) == -1                 # no parameters
    assert plan([(4,)], 0, 0) == -1             # R < 1
    assert plan([(4,)], 65, 0) == -2            # R beyond the kernel argument limit
    assert plan([(4,)], 2, 7) == -1             # unknown layout
    assert plan([(0, 3)], 2, 0) == -1           # empty dimension
    assert plan([(-2,)], 2, 1) == -1
    assert plan([(4,)], 2, 0, ndims=[0]) == -1  # 0-d parameter
    assert plan([(1,) * 9], 2, 0) == -1         # more than 8 dims
    with pytest.raises(F.FsdpError):
        F.Plan([(3,)], 100, "flat")


def test_plan_queries_reject_bad_arguments():
    pg = F.Plan([(5, 2)], 3, "per_param")
    L = F.lib()
    out = (ctypes.c_int64 * 5)()
    assert L.fsdp_plan_param(pg.handle, 1, out) == -1
    assert L.fsdp_plan_param(None, 0, out) == -1
    v = ctypes.c_int64()
    assert L.fsdp_plan_rank_valid(pg.handle, 3, ctypes.byref(v)) == -1
    seg = (ctypes.c_int64 * 4)()
    assert L.fsdp_plan_segments(pg.handle, seg, 0) == -1
    assert L.fsdp_plan_state_bytes_per_rank(None) == -1


def test_page_layout_pins_through_the_library():
    """The FlatParameter offsets and per-GPU counts of the TransformerBlock
    example, read back from the library's plan."""
    from workloads.configs import LINEARS_512
    fl = F.Plan(shapes_of(LINEARS_512), 4, "flat")
    starts = sorted(f0 for _, _, f0, _ in fl.segments())
    assert starts == [0, 786432, 1572864, 2359296] and fl.T == 3145728
    pp = F.Plan(shapes_of(LINEARS_512), 4, "per_param")
    assert pp.S == 786432
    assert pp.comm_ledger(False)["all_gather"] * 2 == 4718592  # 3/4 of 6.3 MB fp16


def test_product_code_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "fully_sharded_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                with open(os.path.join(dirpath, fn)) as f:
                    src = f.read()
                assert "oracle" not in src.lower(), fn


# --------------------------------------------------- work tables, host side
def expand(items, size):
    """Items (dst, src, len) -> per-destination source index (-1 padding),
    checking that they tile [0, size) in order."""
    m = np.full(size, -2, np.int64)
    pos = 0
    for dst, src, n in items:
        assert dst == pos and n > 0
        m[dst:dst + n] = -1 if src < 0 else np.arange(src, src + n)
        pos += n
    assert pos == size
    return m


def oracle_shard_map(po):
    """Oracle layout as a map: shard position r*S+j -> flat index (-1 pad)."""
    m = np.full(po.R * po.S, -1, np.int64)
    for r in range(po.R):
        for f0, s0, n in po.pieces(r):
            m[r * po.S + s0:r * po.S + s0 + n] = np.arange(f0, f0 + n)
    return m


@pytest.mark.parametrize("R", [1, 2, 3, 5, 8])
def test_work_items_tile_both_spaces_like_the_oracle(R):
    rng = np.random.default_rng(40 + R)
    for trial in range(15):
        shapes = [(int(rng.integers(1, 3 * R + 3)),) + tuple(int(x) for x in rng.integers(1, 300, int(rng.integers(0, 2))))
                  for _ in range(int(rng.integers(1, 5)))]
        layout = O.FLAT if trial % 2 else O.PER_PARAM
        po = O.plan_layout(shapes, R, layout)
        pg = F.Plan(shapes, R, layout)
        shard = expand(pg.work_items(0), R * po.S)
        want = oracle_shard_map(po)
        np.testing.assert_array_equal(shard, want)
        assert all(n <= 1024 for _, _, n in pg.work_items(0))
        flat = expand(pg.work_items(1), po.T)
        inv = np.full(po.T, -1, np.int64)
        valid = want >= 0
        inv[want[valid]] = np.flatnonzero(valid)
        np.testing.assert_array_equal(flat, inv)
        assert all(n <= 2048 for _, _, n in pg.work_items(1))


@pytest.mark.parametrize("Ra,Rb", [(8, 4), (4, 8), (3, 5), (1, 2), (6, 6)])
def test_resharder_items_match_the_oracle_reshard(Ra, Rb):
    rng = np.random.default_rng(Ra * 100 + Rb)
    for trial in range(10):
        shapes = [(int(rng.integers(1, 3 * max(Ra, Rb) + 3)),) + tuple(int(x) for x in rng.integers(1, 50, int(rng.integers(0, 3))))
                  for _ in range(int(rng.integers(1, 5)))]
        la = O.FLAT if trial % 2 else O.PER_PARAM
        lb = O.PER_PARAM if trial % 3 else O.FLAT
        pa, pb = O.plan_layout(shapes, Ra, la), O.plan_layout(shapes, Rb, lb)
        rs = F.Resharder(F.Plan(shapes, Ra, la), F.Plan(shapes, Rb, lb))
        got = expand(rs.work_items(), Rb * pb.S)
        # the oracle re-shards the source positions' own indices (+1; 0 = pad)
        idx = (np.arange(Ra * pa.S, dtype=np.int64) + 1).reshape(Ra, pa.S)
        idx[O.shard_pack(pa, np.ones(pa.T, np.int64)) == 0] = 0
        want = O.reshard(pa, pb, idx).reshape(-1) - 1
        np.testing.assert_array_equal(got, want)


def test_resharder_rejects_different_units():
    with pytest.raises(F.FsdpError):
        F.Resharder(F.Plan([(4, 2)], 2, "flat"), F.Plan([(4, 3)], 2, "flat"))


def test_header_compiles_as_c99_and_plans_from_plain_c(tmp_path):
    """A plain C99 program includes include/fsdp_mi355x.h, links the library and
    plans the TransformerBlock FlatParameter of the 4-GPU example."""
    import shutil
    gcc = shutil.which("gcc") or shutil.which("cc")
    if gcc is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(F.binding.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", str(exe),
                    "-L", libdir, "-l:libfsdp_mi355x.so", "-Wl,-rpath," + libdir], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    assert out[0] == "T 3145728 S 786432 R 4 segments 4"
    assert out[1:5] == ["offset 0", "offset 786432", "offset 1572864", "offset 2359296"]
    assert out[5] == "all_gather 2359296"
    assert out[6] == f"state_bytes {16 * 786432}"
    assert out[7] == "R=0 -> invalid argument, out NULL"


# Argument checks of the entry points beyond the plan, on the host: every
# check runs before the first device call, so invalid arguments are rejected
# with FSDP_ERR_INVALID_ARG on a machine without a GPU too.  Pointers below
# are plain numbers, disjoint 4 GiB apart, never dereferenced.
def _fake(i, off=0):
    return ctypes.c_void_p((1 << 40) + (i << 32) + off)


def _parr(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*[p.value for p in ptrs])


def test_step_then_gather_checks_arguments_before_any_device_call():
    L = F.lib()
    pa = F.Plan([(64, 8), (8,)], 4, "per_param")
    pb = F.Plan([(32, 8)], 4, "flat")
    hp = F.binding.AdamWHParams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    grads = _parr([_fake(i) for i in range(4)])
    master, m, v, param = _fake(10), _fake(11), _fake(12), _fake(13)
    shards = _fake(20)
    recv = [_fake(30 + i) for i in range(4)]

    def call(step=1, h=hp, plan=pa, nxt=pb, sh=shards, rc=recv, par=param, g=grads):
        return L.fsdp_adamw_step_then_gather(plan.handle if plan else None, ctypes.byref(h), step,
                                             g, 1, master, m, v, par, 1,
                                             nxt.handle if nxt else None, sh, _parr(rc), None)

    assert call(plan=None) == -1
    assert call(nxt=None) == -1
    assert call(step=0) == -1
    assert call(h=F.binding.AdamWHParams(1e-3, 1.0, 0.999, 1e-8, 0.01)) == -1   # beta1 = 1
    assert call(rc=[master] + recv[1:]) == -1          # a receiver is the master
    assert call(rc=[_fake(1, 64)] + recv[1:]) == -1    # a receiver inside gradient 1
    assert call(sh=param) == -1                        # the gather reads what the step writes
    assert call(sh=_fake(13, 16)) == -1                # ... or part of it
    assert call(rc=[recv[0], recv[0]] + recv[2:]) == -1  # two receivers are one buffer
    assert call(par=_fake(13, 1)) == -1                # bf16 parameter not 2-byte aligned
    # valid arguments: the first device call fails without a GPU
    assert call() == -4


def test_step_graph_checks_arguments_without_a_device():
    L = F.lib()
    hp = F.binding.AdamWHParams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    bad = F.binding.AdamWHParams(1e-3, 0.9, 0.999, 0.0, 0.01)       # eps = 0
    g = ctypes.c_void_p(77)
    assert L.fsdp_step_graph_create(ctypes.byref(hp), None) == -1
    assert L.fsdp_step_graph_create(ctypes.byref(bad), ctypes.byref(g)) == -1
    assert g.value is None                     # cleared on error
    assert L.fsdp_step_graph_create(ctypes.byref(hp), ctypes.byref(g)) == -4   # no device
    assert g.value is None
    L.fsdp_step_graph_destroy(None)
    n, a = ctypes.c_int64(), ctypes.c_int64()
    assert L.fsdp_step_graph_info(None, ctypes.byref(n), ctypes.byref(a)) == -1
    assert L.fsdp_step_graph_launch(None, 1, None) == -1
    pa = F.Plan([(8,)], 2, "flat")
    assert L.fsdp_step_graph_add_gather(None, pa.handle, _fake(1), 1, _parr([_fake(2), _fake(3)])) == -1
    assert L.fsdp_step_graph_add_adamw_gather(None, pa.handle, _parr([_fake(4), _fake(5)]), 1,
                                              _fake(6), _fake(7), _fake(8), _fake(9), 1,
                                              pa.handle, _fake(10),
                                              _parr([_fake(11), _fake(12)])) == -1


def test_reshard_batch_checks_arguments_before_any_device_call():
    L = F.lib()
    a, b = F.Plan([(40, 3)], 4, "per_param"), F.Plan([(40, 3)], 3, "flat")
    rs = F.Resharder(a, b)
    srcs = [_fake(i) for i in range(3)]
    dsts = [_fake(10 + i) for i in range(3)]

    def call(s, d, n=None):
        return L.fsdp_reshard_batch(rs.handle, len(s) if n is None else n, _parr(s), _parr(d), 0,
                                    None)

    assert call(srcs, dsts, n=0) == -1
    assert call([_fake(i) for i in range(65)], [_fake(100 + i) for i in range(65)]) == -2
    assert call(srcs, [dsts[0], dsts[0], dsts[2]]) == -1        # two destinations are one
    assert call(srcs, [srcs[1]] + dsts[1:]) == -1               # a destination is a source
    assert call(srcs, [_fake(10, 2)] + dsts[1:]) == -1          # fp32 misaligned
    assert call(srcs, dsts) == -4                               # valid: no device here


def test_units_beyond_one_launch_grid_are_refused():
    """A launch holds at most 2^32 - 1 lanes per grid dimension: 16,777,215
    workgroups of 256 lanes, so 16,777,215 work items of 1024 shard
    elements.  Larger units are refused when planned, before any table is
    built; the largest accepted size is checked through the item count."""
    L = F.lib()
    limit = 0xFFFFFFFF // 256

    def status(shapes, R, layout):
        nd = [len(s) for s in shapes]
        flat = [d for s in shapes for d in s]
        h = ctypes.c_void_p()
        st = L.fsdp_plan_layout(len(nd), (ctypes.c_int32 * len(nd))(*nd),
                                (ctypes.c_int64 * len(flat))(*flat), R, layout, ctypes.byref(h))
        if st == 0:
            L.fsdp_plan_destroy(h)
        return st

    over = limit * 1024 + 1
    assert status([(over,)], 1, 1) == -2                    # flat, R = 1
    assert status([(over // 8 + 1, 8)], 8, 0) == -2        # per-parameter rows, R = 8
    assert status([(3, over // 3 + 1)], 64, 0) == -2       # padding counts too: S = row
    with pytest.raises(F.FsdpError):
        F.Plan([(over,)], 1, "flat")
    # exactly the limit is still planned (two tables of 16,777,215 items,
    # about 800 MB of host memory)
    assert status([(limit * 1024,)], 1, 1) == 0


def test_c_driver_refuses_bad_input_before_any_device_call(tmp_path):
    """The plain-C driver of the GPU tests (built with the library) checks
    its input files before it touches the GPU."""
    exe = os.path.join(ROOT, "tests", "c", "step_from_c")
    assert os.path.exists(exe), "build the library first: python -m fully_sharded_amd._build"
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 1 and "usage" in out.stderr
    out = subprocess.run([exe, str(tmp_path / "missing")], capture_output=True, text=True,
                         timeout=60)
    assert out.returncode == 1 and "shape.txt" in out.stderr
    (tmp_path / "shape.txt").write_text("2 0 1\n0\n")
    out = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 1 and "bad ndims" in out.stderr


def test_noalloc_step_refuses_a_table_beyond_its_buffer_without_a_device():
    """The no-allocation AdamW entry point keeps the work table in a 1 MiB
    static buffer (43,690 items): a larger plan is refused before the other
    arguments are looked at; a fitting plan goes on to the argument checks."""
    L = F.lib()
    h = F.binding.AdamWHParams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    arr = (ctypes.c_void_p * 1)(None)
    big = F.Plan([(50_000_000,)], 1, "flat")
    assert len(big.work_items(0)) == 48829
    assert L.fsdp_adamw_shard_step_noalloc(big.handle, ctypes.byref(h), 1, arr, 1, 1,
                                           None, None, None, None, 1, None) == -2
    fits = F.Plan([(44_000_000,)], 1, "flat")
    assert len(fits.work_items(0)) <= 43690
    assert L.fsdp_adamw_shard_step_noalloc(fits.handle, ctypes.byref(h), 1, arr, 1, 1,
                                           None, None, None, None, 1, None) == -1
    assert L.fsdp_adamw_shard_step_noalloc(None, ctypes.byref(h), 1, arr, 1, 1,
                                           None, None, None, None, 1, None) == -1
