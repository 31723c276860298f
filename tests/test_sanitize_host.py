"""The plan, re-shard and argument-check code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the host (no GPU): plan.cpp, abi.cpp and
graph.cpp built with host-side sanitizers and the kernel launchers replaced
by stubs that report no device (tests/c/launch_stub.cpp), linked into
tests/c/sanitize_host.cpp.  It checks random units' plan queries, re-shard
tables and every entry point's argument checks; its plan dumps are compared
with the oracle's layout here.  Any sanitizer report fails the run."""

import os
import subprocess

import numpy as np
import pytest

from oracle import fsdp_oracle as O
from workloads.configs import BLOCK_512, shapes_of

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "fully_sharded_amd", "csrc")
SOURCES = [os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "abi.cpp"),
           os.path.join(CSRC, "graph.cpp"), os.path.join(ROOT, "tests", "c", "launch_stub.cpp"),
           os.path.join(ROOT, "tests", "c", "sanitize_host.cpp")]
# sanitizers on the host code only (device code is compiled as usual)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("no hipcc")
    d = tmp_path_factory.mktemp("sanitize")
    objs = []
    for src in SOURCES:
        obj = str(d / (os.path.basename(src) + ".o"))
        subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                        "-fno-omit-frame-pointer", *SAN, "-I", os.path.join(ROOT, "include"),
                        "-I", CSRC, "-c", src, "-o", obj], check=True, capture_output=True)
        objs.append(obj)
    exe = str(d / "sanitize_host")
    subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN[:4], *objs, "-o", exe,
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
                   check=True, capture_output=True)
    return exe


def run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    out = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=600,
                         env=env)
    assert "Sanitizer" not in out.stderr and "runtime error" not in out.stderr, out.stderr[-4000:]
    assert out.returncode == 0, (out.returncode, out.stdout[-2000:], out.stderr[-4000:])
    return out.stdout


def test_random_units_and_entry_points_under_sanitizers(driver):
    out = run(driver, "random", 3000)
    assert "checked 3000 random units, failures 0" in out


@pytest.mark.parametrize("R,layout", [(4, "per_param"), (3, "per_param"), (4, "flat"),
                                      (3, "flat"), (8, "per_param"), (13, "flat")])
def test_sanitized_plan_dump_matches_the_oracle(driver, R, layout):
    rng = np.random.default_rng(R * 31 + len(layout))
    cases = [shapes_of(BLOCK_512)]
    for _ in range(5):
        cases.append([(int(rng.integers(1, 3 * R + 3)),) +
                      tuple(int(x) for x in rng.integers(1, 40, int(rng.integers(0, 3))))
                      for _ in range(int(rng.integers(1, 6)))])
    for shapes in cases:
        nd = [len(s) for s in shapes]
        dims = [d for s in shapes for d in s]
        out = run(driver, "dump", R, 0 if layout == "per_param" else 1, len(shapes), *nd, *dims)
        lines = out.split("\n")
        T, S = map(int, lines[0].split())
        po = O.plan_layout(shapes, R, layout)
        assert (T, S) == (po.T, po.S)
        got = sorted(tuple(map(int, ln.split())) for ln in lines[1:] if ln.strip())
        want = []
        for r in range(R):
            for f0, s0, n in po.pieces(r):
                if n > 0:
                    want.append((r, s0, f0, n))
        # the library merges pieces adjacent in both spaces; compare per element
        def expand(segs):
            return sorted((r, s0 + i, f0 + i) for r, s0, f0, n in segs for i in range(n))
        assert expand(got) == expand(want)
