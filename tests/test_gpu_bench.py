"""bench.py on the GPU, in-process and briefly: the one JSON line carries the
fields its contract names, with consistent values, for the step on a small
workload and for each widened mode."""

import json
import sys

import pytest

import bench

pytestmark = pytest.mark.gpu


def run_bench(capsys, monkeypatch, *argv):
    monkeypatch.setattr(sys, "argv", ["bench.py", *argv])
    bench.main()
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, lines
    return json.loads(lines[-1])


def test_step_line_contract(capsys, monkeypatch):
    print("[gpu] bench step block512_r4", flush=True)
    d = run_bench(capsys, monkeypatch, "--workload", "block512_r4", "--steps", "4",
                  "--warmup", "1", "--cpu-seconds", "1.0", "--cycle-gib", "0.25",
                  "--sustained-workload", "block512_flat_r4")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 4 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["config"]["workload"] == "block512_r4" and d["config"]["R"] == 4
    # the default schedule is chosen by timing: the line names the choice
    sc = d["config"]["schedule_choice"]
    assert sc["requested"] == "auto" and d["config"]["schedule"] == sc["chosen"]
    assert set(sc["ms_per_step"]) == {"overlap", "serial"}
    # value is the step's parameters over its time
    assert d["value"] == pytest.approx(d["config"]["params"] / (d["ms_per_step"] * 1e-3))
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert rf["achieved"] == pytest.approx(rf["bytes_per_launch"] / (rf["avg_ms"] * 1e-3) / 1e9)
    assert 0 < rf["frac"] < 1
    assert rf["target_frac"] == 0.70 and rf["target_met"] == (rf["frac"] >= 0.70)
    assert rf["kernel"].startswith("k_fused")
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["sample"]
    legs = cb["legs"]
    assert legs["one_core"]["cores"] == 1 and legs["one_core"]["value"] > 0
    assert cb["cores"] == legs["all_cores"]["cores"] >= 1
    assert cb["value"] == legs["all_cores"]["value"]
    assert legs["sustained_workload_chunks"]["value"] > 0
    su = d["sustained"]
    assert su["workload"] == "block512_flat_r4" and su["R"] == 4
    for key in ("fused_rs_adamw", "gather_unflatten"):
        k = su[key]
        assert k["gbps"] == pytest.approx(k["bytes"] / (k["avg_ms"] * 1e-3) / 1e9)
        assert 0 < k["frac"] < 1
    # 4 steps timed in 4 blocks of one: the mean lies between their min and max
    bl = d["ms_per_step_blocks"]
    assert bl["blocks"] == 4 and 0 < bl["min"] <= bl["median"]
    assert bl["min"] <= d["ms_per_step"] * (1 + 1e-6)
    cc = d["plain_copy"]
    assert cc["bytes_per_launch"] == pytest.approx(rf["bytes_per_launch"], rel=1e-4)
    assert cc["achieved"] == pytest.approx(cc["bytes_per_launch"] / (cc["avg_ms"] * 1e-3) / 1e9)
    assert 0 < cc["frac"] < 1
    for name, k in d["kernels"].items():
        if isinstance(k, dict):
            assert k["of_plain_copy"] == pytest.approx(k["gbps"] / k["plain_copy_gbps"]), name
            assert 0 < k["of_plain_copy"] < 2, name


@pytest.mark.parametrize("mode", ["reshard", "accum", "ddp"])
def test_mode_lines(capsys, monkeypatch, mode):
    print(f"[gpu] bench mode {mode}", flush=True)
    extra = ["--to-ranks", "3"] if mode == "reshard" else []
    d = run_bench(capsys, monkeypatch, "--mode", mode, "--workload", "block512_r4",
                  "--steps", "3", "--warmup", "1", "--no-cpu-baseline", *extra)
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["roofline"]["bound"] == "hbm" and 0 < d["roofline"]["frac"] < 1
    assert d["config"]["mode"] == mode
    assert d["plain_copy"]["bytes_per_launch"] == pytest.approx(
        d["roofline"]["bytes_per_launch"], rel=1e-4)
    for name, k in d["kernels"].items():
        assert k["of_plain_copy"] == pytest.approx(k["gbps"] / k["plain_copy_gbps"]), name
