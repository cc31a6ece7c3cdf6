"""Pins for the per-head 3D tile order (oracle/tiles.py), on the CPU."""

import numpy as np
import pytest

from oracle import sla, tiles


def test_is_a_permutation_and_blocks_are_boxes():
    grid, tile = (4, 6, 8), (2, 3, 4)
    perm = tiles.tile_order(grid, tile)
    assert sorted(perm.tolist()) == list(range(4 * 6 * 8))
    b = 2 * 3 * 4
    T, Y, X = grid
    for j in range(len(perm) // b):
        toks = perm[j * b:(j + 1) * b]
        t, y, x = toks // (Y * X), (toks // X) % Y, toks % X
        # a box of exactly the tile's extent, aligned to the tile grid
        assert t.max() - t.min() + 1 == 2 and y.max() - y.min() + 1 == 3 and x.max() - x.min() + 1 == 4
        assert t.min() % 2 == 0 and y.min() % 3 == 0 and x.min() % 4 == 0
        assert len(set(toks.tolist())) == b


def test_row_tiles_reduce_to_raster_order():
    # a tile that spans whole rows keeps the raster order
    assert tiles.tile_order((3, 4, 8), (1, 1, 8)).tolist() == list(range(96))
    assert tiles.tile_order((3, 4, 8), (1, 4, 8)).tolist() == list(range(96))


def test_hand_example():
    # grid 1 x 2 x 4 with 1 x 2 x 2 boxes: [0 1 4 5] then [2 3 6 7]
    assert tiles.tile_order((1, 2, 4), (1, 2, 2)).tolist() == [0, 1, 4, 5, 2, 3, 6, 7]


def test_permute_roundtrip_per_head():
    g = np.random.default_rng(0)
    grid = (2, 4, 8)
    x = g.normal(size=(2, 3, 64, 5))
    shapes = [(1, 4, 8), (2, 2, 4), (2, 4, 2)]
    y = tiles.permute(x, grid, shapes)
    np.testing.assert_array_equal(tiles.unpermute(y, grid, shapes), x)
    np.testing.assert_array_equal(y[:, 1], x[:, 1][:, tiles.tile_order(grid, shapes[1])])


def test_undivided_grid_is_refused():
    with pytest.raises(ValueError):
        tiles.tile_order((3, 4, 8), (2, 4, 8))


def test_attention_is_permutation_equivariant_with_a_dense_map():
    # with every tile critical, permuting tokens permutes the output
    g = np.random.default_rng(1)
    grid, tile = (2, 4, 4), (2, 2, 2)
    q, k, v = (g.normal(size=(1, 1, 32, 4)) for _ in range(3))
    cls = np.full((1, 1, 4, 4), sla.CRITICAL, dtype=np.uint8)
    o_ref = sla.forward(q, k, v, cls, 8)[3]
    qp, kp, vp = (tiles.permute(t, grid, [tile]) for t in (q, k, v))
    o_p = sla.forward(qp, kp, vp, cls, 8)[3]
    np.testing.assert_allclose(tiles.unpermute(o_p, grid, [tile]), o_ref, rtol=1e-12, atol=1e-14)
