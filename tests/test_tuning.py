"""Tile-config machinery on the host: the instance query, the LDS-budget filter, the
descriptor's tile request and the sweep cache (no GPU needed)."""
import os

import pytest

import gemm_epilogue_transformer_tiled_amd as ge
from gemm_epilogue_transformer_tiled_amd import tuning

SHAPES = {ge.GE_TILE_256x256: (256, 256, 0, 256), ge.GE_TILE_256x128_PAIR: (256, 128, 1, 256),
          ge.GE_TILE_128x128: (128, 128, 0, 256), ge.GE_TILE_64x64: (64, 64, 0, 256),
          ge.GE_TILE_128x128_PAIR: (128, 128, 1, 256), ge.GE_TILE_256x256_2W: (256, 256, 0, 512),
          ge.GE_TILE_256x128_PAIR_2W: (256, 128, 1, 512)}


def test_tile_info_of_every_instance():
    assert len(SHAPES) == ge.GE_TILE_COUNT
    for t, (bm, bn, pair, threads) in SHAPES.items():
        i = ge.gemm_epilogue_tile_info(t)
        assert (i.bm, i.bn, i.pairwise, i.threads) == (bm, bn, pair, threads)
        assert 0 < i.lds_bytes <= tuning.LDS_PER_CU
    for bad in (-1, ge.GE_TILE_COUNT):
        with pytest.raises(ge.GemmEpilogueError):
            ge.gemm_epilogue_tile_info(bad)


def _desc(chain, **kw):
    return ge.make_desc(1, 512, 512, 512, ge.make_ops(chain), **kw)


def test_admissible_tiles_match_the_chain_and_the_lds_budget():
    single = _desc([("scale",), ("bias",), ("act", "relu")])
    pair = _desc([("pairwise", "silu")])
    assert tuning.admissible_tiles(single) == [0, 2, 3, 5]
    assert tuning.admissible_tiles(pair) == [1, 4, 6]
    # the two-wave instances only where they apply: K a multiple of two steps (64 bf16, 128 fp8)
    assert tuning.admissible_tiles(ge.make_desc(1, 512, 512, 520, ge.make_ops([("scale",)]))) == [0, 2, 3]
    assert tuning.admissible_tiles(_desc([("scale",)], b_layout=ge.GE_LAYOUT_NK)) == [0, 2, 3, 5]
    f8 = dict(b_layout=ge.GE_LAYOUT_NK, a_type=ge.GE_DT_FP8_E4M3, b_type=ge.GE_DT_FP8_E4M3)
    assert tuning.admissible_tiles(_desc([("scale",)], **f8)) == [0, 2, 3, 5]
    assert tuning.admissible_tiles(ge.make_desc(1, 512, 512, 576, ge.make_ops([("scale",)]), **f8)) == [0, 2, 3]
    # a tighter budget removes the instances that allocate more LDS
    lds = {t: ge.gemm_epilogue_tile_info(t).lds_bytes for t in SHAPES}
    budget = lds[ge.GE_TILE_64x64]
    assert tuning.admissible_tiles(single, budget) == [ge.GE_TILE_64x64]
    assert tuning.admissible_tiles(pair, budget) == []


@pytest.mark.parametrize("chain,tile,want", [
    ([("scale",)], None, ge.GE_OK),
    ([("scale",)], ge.GE_TILE_64x64, ge.GE_OK),
    ([("scale",)], ge.GE_TILE_256x128_PAIR, ge.GE_ERR_INVALID_ARG),    # pairwise instance, plain chain
    ([("pairwise", "silu")], ge.GE_TILE_128x128_PAIR, ge.GE_OK),
    ([("pairwise", "silu")], ge.GE_TILE_128x128, ge.GE_ERR_INVALID_ARG),
])
def test_descriptor_tile_request(chain, tile, want):
    assert ge.gemm_epilogue_validate(_desc(chain, tile=tile)) == want


def test_descriptor_tile_out_of_range():
    d = _desc([("scale",)])
    for bad in (-1, ge.GE_TILE_COUNT + 1):
        d.tile = bad
        assert ge.gemm_epilogue_validate(d) == ge.GE_ERR_INVALID_ARG


def test_cache_round_trip(tmp_path):
    path = os.path.join(tmp_path, "tiles.json")
    c = tuning.TileCache.load(path)
    d1 = _desc([("scale",), ("act", "relu")])
    d2 = _desc([("scale",), ("act", "gelu_tanh")])
    assert c.lookup(d1) is None
    assert c.record(d1, {0: 0.30, 2: 0.20, 3: 0.25}) == 2
    c.save()
    c2 = tuning.TileCache.load(path)
    assert c2.lookup(d1) == 2
    assert c2.lookup(d2) is None                      # another chain, another key
    d3 = ge.make_desc(1, 512, 512, 1024, ge.make_ops([("scale",), ("act", "relu")]))
    assert tuning.signature(d3) != tuning.signature(d1)
