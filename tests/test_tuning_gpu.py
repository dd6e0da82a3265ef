"""The tile-config sweep on the GPU: every admissible instance is timed on the problem, the
fastest is cached, and a plan built from the cache runs that instance and matches the oracle."""
import dataclasses
import os

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

ge = pytest.importorskip("gemm_epilogue_transformer_tiled_amd")
from gemm_epilogue_transformer_tiled_amd import runner, tuning  # noqa: E402
from tests.test_parity_gpu import compare  # noqa: E402

NAMES = {0: "256x256", 1: "256x128", 2: "128x128", 3: "64x64", 4: "128x128"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,shape", [("c2", dict(batch=2, M=512, N=768, K=512)),
                                        ("c3", dict(M=512, N=1024, K=256))])
def test_sweep_caches_the_fastest_instance_and_it_computes_the_same(name, shape, tmp_path):
    w = workloads.WORKLOADS[name].with_shape(**shape)
    inp = workloads.generate(w)
    prob = runner.prepare(w, inp)
    cache = tuning.TileCache.load(os.path.join(tmp_path, "tiles.json"))
    best, timings = runner.tune(prob, cache, steps=5)
    assert sorted(timings) == tuning.admissible_tiles(prob.plan.desc)
    assert all(ms > 0 for ms in timings.values())
    assert best == min(timings, key=timings.get)
    cache.save()
    tuned = runner.prepare(w, inp, cache=tuning.TileCache.load(cache.path))
    assert f"tile={NAMES[best]}" in tuned.plan.describe()
    tuned.run()
    torch.cuda.synchronize()
    compare(w, inp, tuned, f"{name} tuned tile {NAMES[best]}")


@pytest.mark.parametrize("tile", [0, 2, 3])
def test_descriptor_tile_request_runs_that_instance(tile):
    w = dataclasses.replace(workloads.WORKLOADS["c5"]).with_shape(batch=1, M=264, N=136, K=200)
    inp = workloads.generate(w)
    prob = runner.prepare(w, inp, tile=tile)
    assert f"tile={NAMES[tile]}" in prob.plan.describe()
    prob.run()
    torch.cuda.synchronize()
    compare(w, inp, prob, f"c5 requested tile {NAMES[tile]}")
