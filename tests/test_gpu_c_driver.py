"""The C ABI used from plain C: tests/c/step_from_c.c (built with the
library by fully_sharded_amd/_build.py) allocates device memory with the
HIP runtime, packs, gathers, reduce-scatters and takes one fused AdamW step
through the library, and writes every result to files; this test draws the
inputs, runs the program in its own process and checks each output against
the oracle, to the same bars as the tests through the Python binding."""

import os
import subprocess

import numpy as np
import pytest

from oracle import fsdp_oracle as O
from tests.gpu_util import assert_adamw_close, assert_bf16_within_ulp, assert_bitexact
from workloads import gen
from workloads.configs import ADAMW

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c", "step_from_c")


@pytest.mark.parametrize("shapes,R,layout", [
    ([(37, 5), (11,), (6, 2, 3)], 3, "per_param"),
    ([(512, 64), (130,)], 5, "flat"),
    ([(9, 7)], 1, "per_param"),
])
def test_step_driven_from_c(tmp_path, shapes, R, layout):
    assert os.path.exists(DRIVER), f"{DRIVER} is missing: run python -m fully_sharded_amd._build"
    print(f"[gpu] C driver R={R} {layout} {shapes}", flush=True)
    po = O.plan_layout(shapes, R, layout)
    T, S = po.T, po.S
    rng = np.random.default_rng(1234 + R)
    master = rng.uniform(-0.5, 0.5, T).astype(np.float32)
    grads = [gen.to_bf16_bits((rng.standard_normal(T) * 1e-2).astype(np.float32))
             for _ in range(R)]
    lay = 0 if layout == "per_param" else 1
    (tmp_path / "shape.txt").write_text(
        f"{R} {lay} {len(shapes)}\n" + " ".join(str(len(s)) for s in shapes) + "\n"
        + " ".join(str(d) for s in shapes for d in s) + "\n")
    master.tofile(tmp_path / "in_master.f32")
    np.stack(grads).tofile(tmp_path / "in_grads.bf16")

    out = subprocess.run([DRIVER, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert "step_from_c ok" in out.stdout

    def load(name, dt, shape):
        return np.fromfile(tmp_path / name, dtype=dt).reshape(shape)

    mo = O.shard_pack(po, master)
    want_full, _ = O.gather_unflatten(po, O.bf16_rne(mo))
    gathered = load("out_gather.bf16", np.uint16, (R, T))
    for r in range(R):
        assert_bitexact(gathered[r], want_full, f"gather receiver {r}")
    assert_bitexact(load("out_rs.f32", np.float32, (R, S)), O.reduce_scatter_avg(po, grads),
                    "reduce-scatter")
    z = np.zeros((R, S), np.float32)
    p1, m1, v1, param1 = O.shard_step(po, grads, mo, z, z, 1, ADAMW, "bf16")
    got_master = load("out_master.f32", np.float32, (R, S))
    assert_adamw_close(got_master, p1, "master")
    assert_adamw_close(load("out_m.f32", np.float32, (R, S)), m1, "m")
    assert_adamw_close(load("out_v.f32", np.float32, (R, S)), v1, "v")
    got_param = load("out_param.bf16", np.uint16, (R, S))
    assert_bf16_within_ulp(got_param, param1, "param")
    assert_bitexact(got_param, O.bf16_rne(got_master), "param = RNE(master)")
