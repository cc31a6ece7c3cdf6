"""Pins for the oracle's mask recall (oracle/sla.py mask_recall), on the CPU."""

import math

import numpy as np

from oracle import sla


def _case(seed, N=37, d=4, b=8, H=2):
    g = np.random.default_rng(seed)
    q, k = g.normal(size=(1, H, N, d)), g.normal(size=(1, H, N, d))
    nb = sla.num_blocks(N, b)
    cls = g.integers(0, 3, size=(1, H, nb, nb)).astype(np.uint8)
    return q, k, cls, b


def test_everything_kept_is_one_and_nothing_kept_is_zero():
    q, k, cls, b = _case(0)
    full = np.full_like(cls, sla.CRITICAL)
    np.testing.assert_allclose(sla.mask_recall(q, k, full, b), 1.0, rtol=0, atol=1e-14)
    empty = np.zeros_like(cls)
    assert not sla.mask_recall(q, k, empty, b).any()


def test_equals_exp_of_lse_difference():
    # the kept mass is exp(LSE over the kept keys - LSE over all keys); the
    # masked attention and the dense one are separate oracle functions
    q, k, cls, b = _case(1)
    N, d = q.shape[-2], q.shape[-1]
    scale = 1.0 / math.sqrt(d)
    r = sla.mask_recall(q, k, cls, b)
    for h in range(q.shape[1]):
        for i in range(sla.num_blocks(N, b)):
            lo, hi = sla.block_bounds(N, b, i)
            crit = np.nonzero(cls[0, h, i] == sla.CRITICAL)[0]
            _, lse_s = sla.attend_block(q[0, h, lo:hi], k[0, h], k[0, h], crit, b, scale)
            _, lse_d = sla.attend_block(q[0, h, lo:hi], k[0, h], k[0, h], np.arange(cls.shape[-1]),
                                        b, scale)
            np.testing.assert_allclose(r[0, h, lo:hi], np.exp(lse_s - lse_d), rtol=1e-12, atol=0)


def test_monotone_in_the_mask_and_additive_over_disjoint_masks():
    q, k, cls, b = _case(2)
    crit = np.where(cls == sla.CRITICAL, sla.CRITICAL, 0).astype(np.uint8)
    marg = np.where(cls == sla.MARGINAL, sla.CRITICAL, 0).astype(np.uint8)
    both = np.where(cls > 0, sla.CRITICAL, 0).astype(np.uint8)
    rc, rm, rb = (sla.mask_recall(q, k, c, b) for c in (crit, marg, both))
    np.testing.assert_allclose(rc + rm, rb, rtol=1e-12, atol=1e-15)
    assert np.all(rb >= rc - 1e-15) and np.all(rb <= 1 + 1e-12)
    # counting marginal tiles as kept is the same as relabelling them critical
    np.testing.assert_allclose(sla.mask_recall(q, k, cls, b, kept=(sla.CRITICAL, sla.MARGINAL)),
                               rb, rtol=1e-12, atol=1e-15)


def test_hand_example_two_keys():
    # two query tokens against two one-token key blocks with logits 0 and
    # ln 3 (scale 1): keeping the second block keeps 3/4 of the mass
    q = np.array([[[[1.0, 0.0], [1.0, 0.0]]]])
    k = np.array([[[[0.0, 0.0], [math.log(3.0), 0.0]]]])
    cls = np.zeros((1, 1, 2, 2), dtype=np.uint8)
    cls[0, 0, :, 1] = sla.CRITICAL
    r = sla.mask_recall(q, k, cls, 1, scale=1.0)
    np.testing.assert_allclose(r[0, 0], [0.75, 0.75], rtol=1e-15)
