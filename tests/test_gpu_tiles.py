"""GPU per-head 3D tile order (sla_tile_permute) against oracle/tiles.py, and
the whole path run on tile-ordered tokens."""

from fractions import Fraction as F

import numpy as np
import pytest
import torch

import block_sparse_attention_meanpool_amd as sla
from gpu_util import bits_of, check_close, say, to_dev
from oracle import sla as osla
from oracle import tiles as otiles
from synth import generate
from synth.configs import Spec

pytestmark = pytest.mark.gpu

GRID = (4, 8, 16)
SHAPES = [(1, 8, 8), (2, 4, 8), (4, 4, 4)]


def _bits(shape, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal(shape).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("d", [128, 64])
def test_permutation_bit_exact_and_roundtrip(d):
    x = _bits((2, 3, 512, d), 1)
    xd = to_dev(x)
    y = sla.sla_tile_permute(xd, GRID, SHAPES, 64)
    back = sla.sla_tile_permute(y, GRID, SHAPES, 64, inverse=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_of(y), otiles.permute(x, GRID, SHAPES))
    np.testing.assert_array_equal(bits_of(back), x)


def test_path_on_tile_ordered_tokens():
    spec = Spec(501, "tiles", B=1, H=3, N=512, d=128, block=64, kind="fourier", grid=GRID,
                mode="topk", keep=F(1, 4))
    data = generate(spec, repairs=None, threads=1)
    nb = spec.nb
    g = np.random.default_rng(7)
    cls = g.choice(np.array([0, 1, 2], dtype=np.uint8), size=(1, 3, nb, nb), p=[0.5, 0.25, 0.25])
    q, k, v = (sla.sla_tile_permute(to_dev(data[t]), GRID, SHAPES, 64) for t in "qkv")
    out = sla.forward(q, k, v, 64, "sla3", cls=torch.from_numpy(cls).cuda(), o_fp32=True)
    pre = (out["o_s"] + out["o_lin"]).contiguous()
    o = sla.sla_tile_permute(out["o"], GRID, SHAPES, 64, inverse=True)
    torch.cuda.synchronize()
    q64, k64, v64 = (otiles.permute(osla.bf16_to_f64(data[t]), GRID, SHAPES) for t in "qkv")
    o_ref = otiles.unpermute(osla.forward(q64, k64, v64, cls, 64)[3], GRID, SHAPES)
    pre_raster = otiles.unpermute(pre.double().cpu().numpy(), GRID, SHAPES)
    check_close(pre_raster, o_ref, "O via tiles (fp32)")
    np.testing.assert_array_equal(bits_of(o), otiles.unpermute(bits_of(out["o"]), GRID, SHAPES))


def test_permutation_at_long_clip_size():
    grid, shape = (60, 64, 64), (2, 8, 8)
    say("[tiles] one head of a 245,760-token grid, tile 2 x 8 x 8")
    x = _bits((1, 2, 60 * 64 * 64, 128), 3)
    y = sla.sla_tile_permute(to_dev(x), grid, [shape, (4, 4, 8)], 128)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_of(y), otiles.permute(x, grid, [shape, (4, 4, 8)]))
