"""The seeded input generators: deterministic, chunk-consistent, and shaped
as the workloads state (no arithmetic of the method lives here)."""

import numpy as np

from workloads import gen
from workloads.configs import BLOCK_512, GROUP_4096, LINEARS_512, WORKLOADS, shapes_of


def test_host_draws_are_deterministic_and_chunked():
    a = gen.host_normal((1, 2, 3), 3 * gen.CHUNK + 17, 1e-3)
    b = gen.host_normal((1, 2, 3), 3 * gen.CHUNK + 17, 1e-3)
    np.testing.assert_array_equal(a, b)
    # a shorter draw is a prefix: chunk c depends only on (key, c)
    c = gen.host_normal((1, 2, 3), gen.CHUNK + 5, 1e-3)
    np.testing.assert_array_equal(a[:gen.CHUNK + 5], c)
    assert not np.array_equal(a[:100], gen.host_normal((1, 2, 4), 100, 1e-3))
    assert abs(float(np.std(a)) - 1e-3) < 2e-5 and abs(float(np.mean(a))) < 2e-6


def test_masters_follow_the_stated_init():
    wl = WORKLOADS["block512_r4"]
    shapes = shapes_of(wl["units"][0])
    m = gen.host_master(wl, 0, shapes)
    off = 0
    for shape in shapes:
        n = int(np.prod(shape))
        x = m[off:off + n]
        if len(shape) == 1:
            assert np.all(x == 1.0)                       # LayerNorm scale
        else:
            bound = 1.0 / np.sqrt(shape[1])
            assert np.all(np.abs(x) <= bound) and np.abs(x).max() > 0.9 * bound
        off += n
    assert off == m.size


def test_bf16_grads_are_torch_rounded():
    import torch
    wl = WORKLOADS["block512_r4"]
    g = gen.host_grad(wl, 1, 0, 0, 1000)
    f = gen.host_normal((wl["cid"], 1, 0, 0, gen.KIND_GRAD), 1000, wl["grad_sigma"])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(g, want)


def test_workload_shapes():
    assert sum(int(np.prod(s)) for s in shapes_of(BLOCK_512)) == 3146752
    assert sum(int(np.prod(s)) for s in shapes_of(LINEARS_512)) == 3145728
    assert sum(int(np.prod(s)) for s in shapes_of(GROUP_4096)) == 872448000
    assert len(WORKLOADS["model12_r8"]["units"]) == 12
