"""Pins for the oracle's gradients (oracle/grad.py), all on the CPU in fp64.

* Central finite differences of L = sum(O * dO), element by element on a
  tiny ragged case, and along random directions on a larger one; the class
  map is held fixed, so L is smooth in Q, K, V (elu + 1 has a continuous
  first derivative) and the difference quotient matches the gradient to
  about eps^2.
* With every tile critical the softmax branch is dense attention, whose
  gradient torch's autograd gives independently (float64 SDPA on the CPU).
* Each branch's gradient alone, against differences of that branch's output.
"""

import math

import numpy as np
import pytest

from oracle import grad, sla

EPS = 1e-6


def _case(seed, B=1, H=2, N=37, d=4, b=8, pattern="mixed"):
    g = np.random.default_rng(seed)
    q, k, v, d_o = (g.normal(size=(B, H, N, d)) for _ in range(4))
    nb = sla.num_blocks(N, b)
    if pattern == "mixed":
        cls = g.integers(0, 3, size=(B, H, nb, nb)).astype(np.uint8)
        cls[0, 0, 0] = sla.CRITICAL        # everything critical
        cls[0, 0, 1] = sla.MARGINAL        # everything marginal
        cls[0, 0, 2] = sla.SKIP            # nothing at all
        cls[0, 1, 0, :] = sla.SKIP
        cls[0, 1, 0, nb - 1] = sla.MARGINAL  # only the ragged last tile, marginal
        cls[0, 1, 1, :] = sla.SKIP
        cls[0, 1, 1, nb - 1] = sla.CRITICAL  # only the ragged last tile, critical
    elif pattern == "critical":
        cls = np.full((B, H, nb, nb), sla.CRITICAL, dtype=np.uint8)
    else:
        raise ValueError(pattern)
    return q, k, v, d_o, cls, b


def _loss(q, k, v, cls, b, d_o, part=3):
    o_s, _, o_lin, o = sla.forward(q, k, v, cls, b)
    out = {1: o_s, 2: o_lin, 3: o}[part]
    return float((out * d_o).sum())


def elementwise_fd_error(seed=0):
    """Max relative error of every gradient entry against central differences."""
    q, k, v, d_o, cls, b = _case(seed, N=11, d=3, b=4)
    got = grad.backward(q, k, v, cls, b, d_o)
    worst = 0.0
    for t, x in enumerate((q, k, v)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + EPS
            lp = _loss(q, k, v, cls, b, d_o)
            x[idx] = old - EPS
            lm = _loss(q, k, v, cls, b, d_o)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * EPS)
        err = np.abs(got[t] - fd).max() / max(1.0, np.abs(fd).max())
        worst = max(worst, err)
    return worst


def directional_fd_error(seed=1, part=3, branches=("softmax", "linear")):
    """Max relative error of <grad, delta> against the central difference along delta."""
    q, k, v, d_o, cls, b = _case(seed)
    got = grad.backward(q, k, v, cls, b, d_o, branches=branches)
    g = np.random.default_rng(seed + 100)
    worst = 0.0
    for t in range(3):
        for _ in range(3):
            delta = g.normal(size=q.shape)
            xs = [q, k, v]
            plus = [x + EPS * delta if i == t else x for i, x in enumerate(xs)]
            minus = [x - EPS * delta if i == t else x for i, x in enumerate(xs)]
            fd = (_loss(*plus, cls, b, d_o, part) - _loss(*minus, cls, b, d_o, part)) / (2 * EPS)
            an = float((got[t] * delta).sum())
            worst = max(worst, abs(an - fd) / max(1.0, abs(fd)))
    return worst


def dense_autograd_error(seed=2):
    """All tiles critical: the gradient against torch autograd of float64 SDPA."""
    torch = pytest.importorskip("torch")
    q, k, v, d_o, cls, b = _case(seed, N=29, d=8, b=8, pattern="critical")
    got = grad.backward(q, k, v, cls, b, d_o)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=1.0 / math.sqrt(8))
    out.backward(torch.tensor(d_o, dtype=torch.float64))
    worst = 0.0
    for a, t in zip(got, (tq, tk, tv)):
        ref = t.grad.numpy()
        worst = max(worst, np.abs(a - ref).max() / max(1.0, np.abs(ref).max()))
    return worst


def test_elementwise_finite_differences():
    assert elementwise_fd_error() < 1e-7


def test_directional_finite_differences():
    assert directional_fd_error() < 1e-7


@pytest.mark.parametrize("part,branches", [(1, ("softmax",)), (2, ("linear",))])
def test_each_branch_alone(part, branches):
    assert directional_fd_error(seed=3, part=part, branches=branches) < 1e-7


def test_all_critical_equals_dense_autograd():
    assert dense_autograd_error() < 1e-12


def test_empty_rows_get_no_gradient():
    q, k, v, d_o, cls, b = _case(4)
    cls[:] = sla.SKIP
    dq, dk, dv = grad.backward(q, k, v, cls, b, d_o)
    assert not dq.any() and not dk.any() and not dv.any()


def test_dphi_closed_form():
    x = np.array([-3.0, -0.5, 0.0, 1e-12, 2.0])
    np.testing.assert_allclose(grad.dphi(x), [math.exp(-3.0), math.exp(-0.5), 1.0, 1.0, 1.0])


def test_linear_dq_scale_bounds_and_closed_form():
    """The size of the linear dQ's terms bounds |dQ| (triangle inequality), and
    with every value row the same vector c the two terms cancel exactly: dQ = 0
    while the size is zeta (|dO| . |c| + |dO . c|) phi'(q) / w."""
    q, k, v, d_o, cls, b = _case(41)
    dq, _, _ = grad.backward(q, k, v, cls, b, d_o, branches=("linear",))
    scale = grad.linear_dq_scale(q, k, v, cls, b, d_o)
    assert (np.abs(dq) <= scale * (1 + 1e-12) + 1e-15).all()
    assert scale[0, 0, 8:16].min() > 0                    # a fully marginal block
    assert not scale[0, 0, 16:24].any()                   # a block with no marginal tile

    g = np.random.default_rng(42)
    N, d, bb = 20, 3, 4
    q1, k1, d1 = (g.normal(size=(1, 1, N, d)) for _ in range(3))
    c = g.normal(size=d)
    v1 = np.broadcast_to(c, (1, 1, N, d)).copy()
    cls1 = np.full((1, 1, 5, 5), sla.MARGINAL, dtype=np.uint8)
    dq1, _, _ = grad.backward(q1, k1, v1, cls1, bb, d1, branches=("linear",))
    sc1 = grad.linear_dq_scale(q1, k1, v1, cls1, bb, d1)
    a = sla.phi(q1[0, 0])
    zeta = sla.phi(k1[0, 0]).sum(axis=0)
    w = a @ zeta
    want = zeta[None, :] * ((np.abs(d1[0, 0]) @ np.abs(c)) + np.abs(d1[0, 0] @ c))[:, None] \
        / w[:, None] * grad.dphi(q1[0, 0])
    assert np.allclose(sc1[0, 0], want, rtol=1e-12, atol=0)
    assert np.abs(dq1).max() < 1e-12 * sc1.max()


@pytest.mark.parametrize("branches", [("softmax",), ("linear",), ("softmax", "linear")])
def test_sampled_gradients_equal_backward(branches):
    """backward_query_blocks and backward_key_tiles (the samplers used on layers
    too long for backward()) give exactly backward()'s rows: the same
    per-block gradients summed in the same order."""
    q, k, v, d_o, cls, b = _case(11, B=1, H=2, N=301, d=8, b=32)
    nb = sla.num_blocks(301, b)
    cls[0, 0, :, 4] = sla.SKIP             # a key tile no query block lists
    ref = grad.backward(q, k, v, cls, b, d_o, branches=branches)
    for h in range(2):
        one = lambda x: x[0, h]
        rows = grad.backward_query_blocks(one(q), one(k), one(v), cls[0, h], b, one(d_o),
                                          range(nb), branches=branches)
        tiles = grad.backward_key_tiles(one(q), one(k), one(v), cls[0, h], b, one(d_o),
                                        [nb - 1, 0, 4, 5], branches=branches)
        for i, got in rows.items():
            lo, hi = sla.block_bounds(301, b, i)
            np.testing.assert_array_equal(got, ref[0][0, h, lo:hi])
        for j, (dk, dv) in tiles.items():
            lo, hi = sla.block_bounds(301, b, j)
            np.testing.assert_array_equal(dk, ref[1][0, h, lo:hi])
            np.testing.assert_array_equal(dv, ref[2][0, h, lo:hi])
        if h == 0:  # the tile no query block lists receives nothing
            assert not tiles[4][0].any() and not tiles[4][1].any()
