"""Per-head 3D token tiles (Veda article, context: heads and layers get their
own tile shapes).  TEST INFRASTRUCTURE ONLY (see the package header).

Tokens of a (T, Y, X) latent grid arrive in raster order n = (t Y + y) X + x.
A tile shape (bt, by, bx) with T, Y, X divisible by bt, by, bx cuts the grid
into boxes; the tile order lists the boxes in raster order of their box index
and, inside each box, its tokens in raster order.  Blocks of bt*by*bx
consecutive tokens of that order are the boxes, which the path then pools,
classifies and attends over unchanged.  (Reading: the pages do not say how a
grid that the tile shape does not divide is handled; it is not supported.)
"""

import numpy as np


def tile_order(grid, tile):
    """perm with perm[p] = raster index of the token at tile-order position p."""
    T, Y, X = grid
    bt, by, bx = tile
    if T % bt or Y % by or X % bx:
        raise ValueError(f"tile {tile} does not divide grid {grid}")
    perm = []
    for ti in range(T // bt):
        for yi in range(Y // by):
            for xi in range(X // bx):
                for dt in range(bt):
                    for dy in range(by):
                        for dx in range(bx):
                            t, y, x = ti * bt + dt, yi * by + dy, xi * bx + dx
                            perm.append((t * Y + y) * X + x)
    return np.array(perm, dtype=np.int64)


def permute(x, grid, tiles):
    """x [B, H, N, ...] in raster order -> tile order, head h with tiles[h]."""
    out = np.empty_like(x)
    for h, tile in enumerate(tiles):
        out[:, h] = x[:, h][:, tile_order(grid, tile)]
    return out


def unpermute(x, grid, tiles):
    """Inverse of permute."""
    out = np.empty_like(x)
    for h, tile in enumerate(tiles):
        out[:, h][:, tile_order(grid, tile)] = x[:, h]
    return out
