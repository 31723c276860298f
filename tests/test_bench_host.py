"""Host logic of bench.py (no GPU): the counter summary that turns two
rocprofv3 --pmc CSVs into HBM bytes per launch, the traffic file's
validity check, the launch count per step, and the buffer carving rule."""

import argparse
import csv
import json

import pytest
import torch

import bench
import fully_sharded_amd as F
from workloads.configs import BLOCK_512, shapes_of

FUSED = "void fsdp::(anonymous namespace)::k_fused<unsigned short, unsigned short, 8>(Work const*)"
PAIR = ("void fsdp::(anonymous namespace)::k_fused_gather<unsigned short, unsigned short, 8>"
        "(Work const*)")
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::copy_kernel>(int)"


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})
        # another counter in the same file is ignored
        w.writerow({"Kernel_Name": FUSED, "Counter_Name": "GRBM_COUNT", "Counter_Value": 1})


@pytest.fixture
def traffic_dir(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_path",
                        lambda wl, key, mode="step": str(tmp_path / f"traffic_{wl}_{key}.json"))
    return tmp_path


def test_counter_summary_scales_by_the_calibration_copy(traffic_dir, capsys):
    fetch, write = traffic_dir / "f.csv", traffic_dir / "w.csv"
    gib_kib = float(1 << 20)
    # FETCH_SIZE reads half of what the 1 GiB copy moves, WRITE_SIZE all of
    # it; a larger set-up copy comes first in the run and is not the
    # calibration (the calibration is the run's last 10 copies)
    calib = bench.CALIB_TIMED
    write_csv(fetch, "FETCH_SIZE", [(COPY, 0.8 * gib_kib), (FUSED, 100.0), (FUSED, 102.0),
                                    (PAIR, 300.0)] + [(COPY, gib_kib / 2)] * (3 + calib))
    write_csv(write, "WRITE_SIZE", [(COPY, 1.6 * gib_kib), (FUSED, 50.0), (FUSED, 50.0),
                                    (PAIR, 90.0)] + [(COPY, gib_kib)] * (3 + calib))
    bench.summarise_counters(str(fetch), str(write), "wl")
    fused = json.loads((traffic_dir / "traffic_wl_fused.json").read_text())
    pair = json.loads((traffic_dir / "traffic_wl_fused_gather.json").read_text())
    assert fused["fetch_scale"] == pytest.approx(2.0) and fused["write_scale"] == pytest.approx(1.0)
    # the k_fused rows only: the k_fused_gather dispatch is not mixed in
    assert fused["fetch_kib_per_launch"] == pytest.approx(101.0)
    assert fused["bytes_per_launch"] == pytest.approx((101.0 * 2 + 50.0) * 1024)
    assert pair["dispatches"] == {"FETCH_SIZE": 1, "WRITE_SIZE": 1}
    assert pair["bytes_per_launch"] == pytest.approx((300.0 * 2 + 90.0) * 1024)
    assert fused["kernel_src_sha"] == bench.kernel_src_hash()


def test_counter_summary_refuses_copies_that_are_not_the_calibration(traffic_dir):
    fetch, write = traffic_dir / "f.csv", traffic_dir / "w.csv"
    gib_kib = float(1 << 20)
    mixed = [(COPY, gib_kib / 2)] * (bench.CALIB_TIMED - 1) + [(COPY, gib_kib)]
    write_csv(fetch, "FETCH_SIZE", [(FUSED, 100.0)] + mixed)
    write_csv(write, "WRITE_SIZE", [(FUSED, 50.0)] + mixed)
    with pytest.raises(SystemExit):
        bench.summarise_counters(str(fetch), str(write), "wl")


def test_counter_summary_needs_the_calibration_copy(traffic_dir):
    fetch, write = traffic_dir / "f.csv", traffic_dir / "w.csv"
    write_csv(fetch, "FETCH_SIZE", [(FUSED, 100.0)])
    write_csv(write, "WRITE_SIZE", [(FUSED, 50.0)])
    with pytest.raises(SystemExit):
        bench.summarise_counters(str(fetch), str(write), "wl")


def test_traffic_is_dropped_once_the_kernels_change(traffic_dir, monkeypatch):
    path = traffic_dir / "traffic_wl_fused.json"
    path.write_text(json.dumps({"kernel_src_sha": bench.kernel_src_hash(),
                                "bytes_per_launch": 123.0}))
    assert bench.load_traffic("wl", "fused") == 123.0
    assert bench.load_traffic("other", "fused") is None
    monkeypatch.setattr(bench, "kernel_src_hash", lambda: "changed")
    assert bench.load_traffic("wl", "fused") is None


class _Unit:
    def __init__(self, plan):
        self.plan = plan


def test_launches_per_step_by_schedule():
    blk = F.Plan(shapes_of(BLOCK_512), 8, "per_param")          # 3,073 work items
    big = F.Plan([(65537 * 1024,)], 8, "flat")                  # > 65,536 work items
    assert len(blk.work_items(0)) <= 65536 < len(big.work_items(0))
    units = [_Unit(blk)] * 12
    a = argparse.Namespace
    assert bench.launches_per_step(a(schedule="serial", gathers_per_step=1), units) == 24
    assert bench.launches_per_step(a(schedule="serial", gathers_per_step=2), units) == 36
    assert bench.launches_per_step(a(schedule="graph", gathers_per_step=1), units) == 25
    # gather(0), 11 pair launches, the last step
    assert bench.launches_per_step(a(schedule="overlap", gathers_per_step=1), units) == 13
    # 12 forward gathers, the last unit's re-gather, 11 pairs, step(0)
    assert bench.launches_per_step(a(schedule="overlap", gathers_per_step=2), units) == 25
    # long steps keep their own launch
    mixed = [_Unit(big), _Unit(blk), _Unit(big)]
    assert bench.launches_per_step(a(schedule="overlap", gathers_per_step=1), mixed) == 1 + 2 + 1 + 1


def test_rows_stagger_strides_that_are_multiples_of_4k():
    a = bench.rows(3, 1024, torch.float32, "cpu")          # 4 KiB per row -> stride + 256 B
    assert a[1].data_ptr() - a[0].data_ptr() == 4096 + 256
    b = bench.rows(3, 1000, torch.float32, "cpu")          # 4,000 B -> 4,096 B: + 256 B too
    assert b[1].data_ptr() - b[0].data_ptr() == 4096 + 256
    c = bench.rows(2, 100, torch.bfloat16, "cpu")          # 200 B -> 256 B
    assert c[1].data_ptr() - c[0].data_ptr() == 256
    assert all(t.numel() == 1024 for t in a) and all(t.numel() == 100 for t in c)


def test_kernel_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "fully_sharded_amd" / "csrc"
    src.mkdir(parents=True)
    files = ("kernels.hip", "kernels.hpp", "plan.cpp", "abi.cpp")
    for f in files:
        (src / f).write_text("int f() { return 1; }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_src_hash()
    (src / "kernels.hip").write_text("// a comment\nint f() {  /* more */ return 1; }\n\n")
    assert bench.kernel_src_hash() == h0
    (src / "kernels.hip").write_text("int f() { return 2; }\n")
    assert bench.kernel_src_hash() != h0


def test_step_blocks_cover_the_timed_steps():
    for steps in (1, 3, 4, 10, 199, 200):
        b = bench.step_blocks(steps)
        assert b[0] == 0 and b[-1] == steps and len(b) - 1 == min(10, steps)
        sizes = [y - x for x, y in zip(b, b[1:])]
        assert min(sizes) >= 1 and max(sizes) - min(sizes) <= 1


def test_plain_copy_sizes():
    assert bench.plain_copy_bytes(188805120) == 188805120
    assert bench.plain_copy_bytes(188805121) == 188805120
    assert bench.plain_copy_bytes(100) == 8192
    assert bench.plain_copy_bytes(36642816000) == 4 << 30


def test_plan_layout_timing_on_the_host():
    from workloads.configs import WORKLOADS
    t = bench.time_plan_layout(WORKLOADS["model12_r8"], budget_s=0.05)
    assert t["plans"] == 1 and t["repeats"] >= 1 and t["ms"] > 0


def test_more_than_one_gpu_exits_with_a_message():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr
