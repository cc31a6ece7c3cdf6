"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a closed
form, a brute-force enumeration, a textbook/library routine for a special
case, or an invariant.  The pinned steps:

* mean pooling of Q and K over blocks (SLA post, "what the idea is";
  NABLA post, point 2);
* pooled softmax over key blocks and the 1 - thr cumulative cut (NABLA post,
  points 2-3);
* top-k over key tiles (Veda article, "what happened");
* the three-way split and the linear branch (SLA post, "what the idea is");
* softmax attention restricted to the kept blocks (all three pages).
"""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import sla


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- bf16 decode

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3FC0, 0x0000, 0x8000, 0x7F80, 0x3E80, 0x4049, 0x0001],
                    dtype=np.uint16)
    want = [1.0, -2.0, 1.5, 0.0, -0.0, math.inf, 0.25, 3.140625, 2.0 ** -133]
    got = sla.bf16_to_f64(bits)
    assert list(got) == want


# ---------------------------------------------------------------- pooling

def test_pool_constant_blocks_give_the_constant():
    b, nb, d = 8, 5, 3
    vals = rng(0).standard_normal((nb, d))
    x = np.repeat(vals, b, axis=0)
    np.testing.assert_allclose(sla.pool(x, b), vals, rtol=4e-16, atol=0)


def test_pool_block_of_one_is_identity():
    x = rng(1).standard_normal((2, 3, 7, 4))
    np.testing.assert_array_equal(sla.pool(x, 1), x)


def test_pool_partial_last_block_uses_valid_tokens_only():
    # N = 5, b = 2: blocks {0,1}, {2,3}, {4}; the last mean is the lone token itself.
    x = np.array([[1.0, 0.0], [3.0, 2.0], [5.0, 5.0], [7.0, -1.0], [10.0, 4.0]])
    want = np.array([[2.0, 1.0], [6.0, 2.0], [10.0, 4.0]])
    np.testing.assert_array_equal(sla.pool(x, 2), want)


def test_pool_is_linear():
    g = rng(2)
    x, y = g.standard_normal((11, 3)), g.standard_normal((11, 3))
    np.testing.assert_allclose(sla.pool(2.0 * x - 3.0 * y, 4), 2.0 * sla.pool(x, 4) - 3.0 * sla.pool(y, 4),
                               rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- pooled scores

def test_pooled_score_equals_mean_of_token_pair_scores():
    # Bilinearity: qbar_i . kbar_j is the mean over the block pair of q_m . k_n.
    g = rng(3)
    N, b, d = 10, 4, 3
    q, k = g.standard_normal((N, d)), g.standard_normal((N, d))
    s = sla.pooled_scores(sla.pool(q, b), sla.pool(k, b), 0.5)
    nb = 3
    for i in range(nb):
        for j in range(nb):
            qi = range(i * b, min(i * b + b, N))
            kj = range(j * b, min(j * b + b, N))
            tot = 0.0
            for m in qi:
                for n in kj:
                    tot += sum(q[m, c] * k[n, c] for c in range(d))
            assert s[i, j] == pytest.approx(0.5 * tot / (len(qi) * len(kj)), rel=1e-12, abs=1e-12)


def test_pooled_scores_orientation():
    # Rows are query blocks, columns key blocks.
    qp = np.array([[1.0, 0.0], [0.0, 0.0]])
    kp = np.array([[0.0, 0.0], [0.0, 0.0], [3.0, 0.0]])
    s = sla.pooled_scores(qp, kp, 1.0)
    assert s.shape == (2, 3)
    assert s[0, 2] == 3.0 and s[0, :2].tolist() == [0.0, 0.0] and not s[1].any()


# ---------------------------------------------------------------- counts (R4)

@pytest.mark.parametrize("frac,nkb,want", [
    (Fraction(1, 4), 16, 4), (Fraction(5, 100), 256, 13), (Fraction(5, 100), 591, 30),
    (Fraction(5, 100), 1920, 96), (Fraction(10, 100), 1920, 192), (Fraction(1, 1000), 16, 1),
])
def test_count_from_fraction(frac, nkb, want):
    assert sla.count_from_fraction(frac, nkb) == want


def test_split_counts():
    assert sla.split_counts(Fraction(5, 100), Fraction(15, 100), 256) == (13, 39)
    assert sla.split_counts(Fraction(5, 100), Fraction(5, 100), 1920) == (96, 96)
    assert sla.split_counts(Fraction(10, 100), Fraction(5, 100), 1920) == (192, 96)
    assert sla.split_counts(Fraction(1, 2), None, 8) == (4, 0)


# ---------------------------------------------------------------- top-k

def test_topk_brute_force_max_sum_subset():
    g = rng(4)
    for trial in range(30):
        nkb = int(g.integers(2, 9))
        k = int(g.integers(1, nkb + 1))
        s = g.standard_normal(nkb)
        cls = sla.classify_row(s, "topk", k)
        best = max(itertools.combinations(range(nkb), k), key=lambda c: sum(s[list(c)]))
        assert set(np.nonzero(cls == sla.CRITICAL)[0]) == set(best)
        assert set(np.unique(cls)) <= {sla.SKIP, sla.CRITICAL}


def test_topk_ties_prefer_lower_index():
    s = [1.0, 3.0, 3.0, 2.0, 3.0]
    assert np.nonzero(sla.classify_row(s, "topk", 1) == 2)[0].tolist() == [1]
    assert np.nonzero(sla.classify_row(s, "topk", 2) == 2)[0].tolist() == [1, 2]
    assert np.nonzero(sla.classify_row(s, "topk", 4) == 2)[0].tolist() == [1, 2, 3, 4]


def test_order_matches_a_library_sort():
    s = rng(5).standard_normal(40)
    assert sla.descending_order(s).tolist() == sorted(range(40), key=lambda j: (-s[j], j))


# ---------------------------------------------------------------- NABLA cut

def _mass(p, subset):
    return sum(p[j] for j in subset)


def test_cdf_brute_force_minimal_then_maximal_mass():
    g = rng(6)
    for trial in range(40):
        nkb = int(g.integers(1, 11))
        s = g.standard_normal(nkb) * g.uniform(0.2, 3.0)
        thr = float(g.uniform(0.02, 0.6))
        cls = sla.classify_row(s, "cdf", thr=thr)
        kept = set(np.nonzero(cls == sla.CRITICAL)[0])
        e = [math.exp(x) for x in s]
        z = sum(e)
        p = [x / z for x in e]
        feasible = [set(c) for r in range(1, nkb + 1) for c in itertools.combinations(range(nkb), r)
                    if _mass(p, c) >= 1.0 - thr]
        mincard = min(len(c) for c in feasible)
        best = max((c for c in feasible if len(c) == mincard), key=lambda c: _mass(p, c))
        assert kept == best


def test_cdf_invariants():
    g = rng(7)
    for trial in range(40):
        nkb = int(g.integers(2, 64))
        s = g.standard_normal(nkb) * 3
        thr = float(g.uniform(0.01, 0.5))
        cls = sla.classify_row(s, "cdf", thr=thr)
        kept = np.nonzero(cls == sla.CRITICAL)[0]
        p = sla.softmax(s)
        assert p[kept].sum() >= 1.0 - thr
        # dropping the weakest kept block loses the mass requirement
        weakest = kept[np.argmin(s[kept])]
        assert p[kept].sum() - p[weakest] < 1.0 - thr or len(kept) == 1
        # the kept set is a prefix of the descending order
        assert min(s[kept]) >= max(np.delete(s, kept), default=-np.inf)


def test_cdf_uniform_scores_closed_form():
    # four equal blocks carry 1/4 each: mass >= 0.9 needs 4, >= 0.7 needs 3, >= 0.5 needs 2
    s = np.zeros(4)
    assert sla.cdf_count(s, 0.1) == 4
    assert sla.cdf_count(s, 0.3) == 3
    assert sla.cdf_count(s, 0.5) == 2
    assert sla.cdf_count(s, 0.8) == 1


def test_cdf_depends_on_score_scale():
    s = np.array([2.0, 1.0, 0.0, -1.0])
    assert sla.cdf_count(s, 0.1) == 3
    assert sla.cdf_count(4 * s, 0.1) == 1


# ---------------------------------------------------------------- SLA three-way split

def test_sla3_invariants():
    g = rng(8)
    for trial in range(30):
        nkb = int(g.integers(3, 80))
        kc = int(g.integers(1, nkb))
        km = int(g.integers(0, nkb - kc + 1))
        s = g.standard_normal(nkb)
        cls = sla.classify_row(s, "sla3", kc, km)
        crit, marg, skip = (np.nonzero(cls == c)[0] for c in (2, 1, 0))
        assert len(crit) == kc and len(marg) == km and len(skip) == nkb - kc - km
        assert s[crit].min() >= (s[marg].max() if km else -np.inf)
        if km and len(skip):
            assert s[marg].min() >= s[skip].max()
        # the critical set is the top-k_c set
        np.testing.assert_array_equal(crit, np.nonzero(sla.classify_row(s, "topk", kc) == 2)[0])


def test_index_lists_ascending_and_padded():
    cls = np.array([[2, 0, 1, 2, 2], [0, 0, 0, 0, 0]], dtype=np.uint8)
    idx, cnt = sla.index_lists(cls, 2, 4)
    assert idx.tolist() == [[0, 3, 4, -1], [-1, -1, -1, -1]]
    assert cnt.tolist() == [3, 0]
    with pytest.raises(ValueError):
        sla.index_lists(cls, 2, 2)


# ---------------------------------------------------------------- sparse branch

def _dense_reference(q, k, v, scale):
    # An independent route: log-sum-exp from scipy instead of max-subtraction.
    from scipy.special import logsumexp
    logits = scale * (q @ k.T)
    lse = logsumexp(logits, axis=1)
    return np.exp(logits - lse[:, None]) @ v, lse


@pytest.mark.parametrize("N,b,d", [(64, 16, 8), (70, 16, 8), (33, 8, 4)])
def test_all_kept_equals_dense_attention(N, b, d):
    g = rng(9)
    q, k, v = (g.standard_normal((N, d)) for _ in range(3))
    nb = sla.num_blocks(N, b)
    scale = 1.0 / math.sqrt(d)
    for i in range(nb):
        lo, hi = sla.block_bounds(N, b, i)
        o, lse = sla.attend_block(q[lo:hi], k, v, range(nb), b, scale)
        o_ref, lse_ref = _dense_reference(q[lo:hi], k, v, scale)
        np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_all_kept_equals_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    g = rng(10)
    B, H, N, d, b = 1, 2, 96, 16, 32
    q, k, v = (g.standard_normal((B, H, N, d)) for _ in range(3))
    cls = np.full((B, H, 3, 3), sla.CRITICAL, dtype=np.uint8)
    o_s, lse, o_lin, o = sla.forward(q, k, v, cls, b)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(o_s, ref, rtol=1e-12, atol=1e-12)
    assert not o_lin.any()
    np.testing.assert_array_equal(o, o_s)


def _brute_token_attention(q, k, v, keep_tok, scale):
    """Token-level masked softmax with explicit -inf entries, in plain loops."""
    r, d = len(q), len(q[0])
    out = []
    for m in range(r):
        logits = []
        for n in range(len(k)):
            if keep_tok[n]:
                logits.append(scale * sum(q[m][c] * k[n][c] for c in range(d)))
            else:
                logits.append(-math.inf)
        mx = max(logits)
        if mx == -math.inf:
            out.append([0.0] * len(v[0]))
            continue
        w = [math.exp(x - mx) for x in logits]
        z = sum(w)
        out.append([sum(w[n] * v[n][c] for n in range(len(k))) / z for c in range(len(v[0]))])
    return np.array(out)


@pytest.mark.parametrize("b", [1, 2, 4])
def test_two_by_two_block_grid_all_masks(b):
    g = rng(11 + b)
    N, d = 2 * b, 4
    for head in range(2):
        q, k, v = (g.standard_normal((N, d)) for _ in range(3))
        for mask in range(16):
            cls = np.array([[(mask >> (2 * i + j)) & 1 for j in range(2)] for i in range(2)],
                           dtype=np.uint8) * sla.CRITICAL
            o_s, lse, o_lin, o = sla.forward(q[None, None], k[None, None], v[None, None], cls[None, None], b)
            for i in range(2):
                keep_tok = [bool(cls[i, n // b]) for n in range(N)]
                want = _brute_token_attention(q[i * b:(i + 1) * b].tolist(), k.tolist(), v.tolist(),
                                              keep_tok, 1.0 / math.sqrt(d))
                np.testing.assert_allclose(o_s[0, 0, i * b:(i + 1) * b], want, rtol=1e-12, atol=1e-12)
                if not cls[i].any():
                    assert np.all(lse[0, 0, i * b:(i + 1) * b] == -np.inf)


def test_sparse_invariants():
    g = rng(12)
    N, b, d = 80, 16, 8
    q, k, v = (g.standard_normal((N, d)) for _ in range(3))
    kept = [4, 1, 3]
    toks = np.concatenate([np.arange(j * b, min(j * b + b, N)) for j in kept])
    o, lse, p = sla.attend_block(q[:b], k, v, kept, b, 0.3, return_p=True)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(o >= v[toks].min(axis=0) - 1e-12) and np.all(o <= v[toks].max(axis=0) + 1e-12)
    # the order of the kept list does not matter
    o2, lse2 = sla.attend_block(q[:b], k, v, sorted(kept), b, 0.3)
    np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-13)
    # constant V gives constant O
    oc, _ = sla.attend_block(q[:b], k, np.full_like(v, 1.75), kept, b, 0.3)
    np.testing.assert_allclose(oc, 1.75, rtol=1e-14)
    # LSE is the log of the normaliser
    logits = 0.3 * q[:b] @ k[toks].T
    np.testing.assert_allclose(lse, np.log(np.exp(logits).sum(axis=1)), rtol=1e-12)


def test_sparse_skips_tokens_past_the_end():
    # the last block holds 3 tokens; the attention must run over exactly them
    g = rng(13)
    N, b, d = 11, 4, 3
    q, k, v = (g.standard_normal((N, d)) for _ in range(3))
    o, _ = sla.attend_block(q[:2], k, v, [2], b, 1.0)
    w = np.exp(q[:2] @ k[8:11].T)
    np.testing.assert_allclose(o, (w / w.sum(1, keepdims=True)) @ v[8:11], rtol=1e-13)


# ---------------------------------------------------------------- linear branch

def test_phi_closed_form_and_elu():
    x = np.array([-np.inf, -1.0, 0.0, 0.5, 1.0, 3.0])
    np.testing.assert_array_equal(sla.phi(x), [0.0, math.exp(-1.0), 1.0, 1.5, 2.0, 4.0])
    torch = pytest.importorskip("torch")
    y = rng(14).standard_normal(1000) * 4
    np.testing.assert_allclose(sla.phi(y), torch.nn.functional.elu(torch.from_numpy(y)).numpy() + 1.0,
                               rtol=1e-15, atol=1e-15)
    assert np.all(sla.phi(y) > 0)


def test_linear_constant_v_gives_constant():
    g = rng(15)
    N, b, d = 64, 16, 8
    q, k = g.standard_normal((N, d)), g.standard_normal((N, d))
    o = sla.linear_block(q[:b], k, np.full((N, d), -0.625), [0, 2, 3], b)
    np.testing.assert_allclose(o, -0.625, rtol=1e-14)


def test_linear_equals_token_quadratic_form():
    # Associativity: phi(q)^T (sum phi(k) v^T) / phi(q).sum phi(k) equals the
    # weighted mean of v with weights phi(q) . phi(k), written out in loops.
    g = rng(16)
    N, b, d = 13, 4, 3
    q, k, v = (g.standard_normal((N, d)) for _ in range(3))
    marg = [3, 1]
    o = sla.linear_block(q[:b], k, v, marg, b)
    toks = [n for j in marg for n in range(j * b, min(j * b + b, N))]
    for m in range(b):
        pq = [math.exp(x) if x <= 0 else x + 1 for x in q[m]]
        w = []
        for n in toks:
            pk = [math.exp(x) if x <= 0 else x + 1 for x in k[n]]
            w.append(sum(a * c for a, c in zip(pq, pk)))
        want = [sum(w[t] * v[n][c] for t, n in enumerate(toks)) / sum(w) for c in range(d)]
        np.testing.assert_allclose(o[m], want, rtol=1e-12)


def test_linear_is_linear_in_v_and_empty_is_zero():
    g = rng(17)
    N, b, d = 32, 8, 4
    q, k, v1, v2 = (g.standard_normal((N, d)) for _ in range(4))
    a = sla.linear_block(q[:b], k, 2 * v1 + v2, [1, 2], b)
    np.testing.assert_allclose(a, 2 * sla.linear_block(q[:b], k, v1, [1, 2], b)
                               + sla.linear_block(q[:b], k, v2, [1, 2], b), rtol=1e-12, atol=1e-12)
    assert not sla.linear_block(q[:b], k, v1, [], b).any()


# ---------------------------------------------------------------- whole forward

def test_forward_three_way_sums_branches():
    g = rng(18)
    B, H, N, d, b = 1, 2, 50, 8, 8
    q, k, v = (g.standard_normal((B, H, N, d)) for _ in range(3))
    cls, s, qp, kp = sla.class_map(q, k, b, "sla3", keep=Fraction(2, 7), marg=Fraction(3, 7))
    assert (cls == 2).sum(-1)[0].tolist() == [[2] * 7] * 2
    assert (cls == 1).sum(-1)[0].tolist() == [[3] * 7] * 2
    o_s, lse, o_lin, o = sla.forward(q, k, v, cls, b)
    np.testing.assert_array_equal(o, o_s + o_lin)
    rows = sla.forward_rows(q, k, v, cls, b, [(0, 1, 6)])
    np.testing.assert_array_equal(rows[(0, 1, 6)][3], o[0, 1, 48:50])


def test_class_map_scale_default_and_modes():
    g = rng(19)
    q, k = g.standard_normal((1, 1, 64, 16)), g.standard_normal((1, 1, 64, 16))
    cls, s, qp, kp = sla.class_map(q, k, 8, "topk", keep=Fraction(1, 4))
    np.testing.assert_allclose(s, (qp @ np.swapaxes(kp, -1, -2)) / 4.0, rtol=1e-13)
    assert ((cls == 2).sum(-1) == 2).all()
    cls2, *_ = sla.class_map(q, k, 8, "maskin", keep=Fraction(1, 4), marg=Fraction(1, 4))
    np.testing.assert_array_equal(cls2 == 2, cls == 2)
    assert ((cls2 == 1).sum(-1) == 2).all()
