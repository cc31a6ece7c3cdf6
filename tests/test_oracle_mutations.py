"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin fails.

Each mutant replaces one oracle function with a subtly wrong variant (a
dropped term, a wrong scale, a flipped comparison, a transposed operand, a
wrong tie order).  The pins in test_oracle_pins.py must reject every one.
"""

import math

import numpy as np
import pytest

import test_oracle_pins as pins
from oracle import sla

_orig = {name: getattr(sla, name) for name in
         ("pool", "pooled_scores", "descending_order", "cdf_count", "attend_block", "phi",
          "linear_block", "classify_row")}


def _pool_divides_by_b(x, b):
    N = x.shape[-2]
    nb = sla.num_blocks(N, b)
    out = np.empty(x.shape[:-2] + (nb, x.shape[-1]))
    for j in range(nb):
        lo, hi = sla.block_bounds(N, b, j)
        out[..., j, :] = x[..., lo:hi, :].sum(axis=-2) / b
    return out


def _scores_transposed(qp, kp, scale):
    return scale * np.matmul(kp, np.swapaxes(qp, -1, -2))


def _order_ties_to_higher(s_row):
    s = np.asarray(s_row, dtype=np.float64)
    return np.array(sorted(range(len(s)), key=lambda j: (-s[j], -j)))


def _cdf_strict(s_row, thr):
    order = sla.descending_order(s_row)
    p = sla.softmax(s_row)
    mass = 0.0
    for m, j in enumerate(order, start=1):
        mass += p[j]
        if mass > 1.0 - thr:
            return m
    return len(order)


def _attend_scale_squared(q_rows, k, v, kept_blocks, b, scale, return_p=False):
    return _orig["attend_block"](q_rows, k, v, kept_blocks, b, scale * scale, return_p)


def _attend_values_from_keys(q_rows, k, v, kept_blocks, b, scale, return_p=False):
    return _orig["attend_block"](q_rows, k, k, kept_blocks, b, scale, return_p)


def _attend_no_renormalise(q_rows, k, v, kept_blocks, b, scale, return_p=False):
    res = _orig["attend_block"](q_rows, k, v, kept_blocks, b, scale, True)
    o, lse, p = res
    # weights normalised over a full block count instead of the kept keys
    o = o * (len(kept_blocks) / max(1, len(kept_blocks) + 1))
    return (o, lse, p) if return_p else (o, lse)


def _phi_plain_elu(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x, np.exp(np.minimum(x, 0.0)) - 1.0)


def _phi_relu_plus_one(x):
    return np.maximum(np.asarray(x, dtype=np.float64), 0.0) + 1.0


def _linear_unnormalised(q_rows, k, v, marg_blocks, b):
    N = k.shape[0]
    toks = sla._tokens_of(marg_blocks, N, b)
    if len(toks) == 0:
        return np.zeros((q_rows.shape[0], v.shape[1]))
    return sla.phi(q_rows) @ (sla.phi(k[toks]).T @ v[toks]) / len(toks)


def _linear_state_transposed(q_rows, k, v, marg_blocks, b):
    N = k.shape[0]
    toks = sla._tokens_of(marg_blocks, N, b)
    if len(toks) == 0:
        return np.zeros((q_rows.shape[0], v.shape[1]))
    pk = sla.phi(k[toks])
    state = (pk.T @ v[toks]).T
    pq = sla.phi(q_rows)
    return (pq @ state) / (pq @ pk.sum(axis=0))[:, None]


def _sla3_marginal_from_bottom(s_row, mode, kc=0, km=0, thr=None):
    cls = _orig["classify_row"](s_row, mode, kc, km, thr)
    if mode == "sla3" and km:
        order = sla.descending_order(s_row)
        cls[order[kc:kc + km]] = sla.SKIP
        cls[order[len(order) - km:]] = sla.MARGINAL
    return cls


MUTANTS = [
    ("pool", _pool_divides_by_b, [pins.test_pool_partial_last_block_uses_valid_tokens_only]),
    ("pooled_scores", _scores_transposed, [pins.test_pooled_scores_orientation]),
    ("descending_order", _order_ties_to_higher, [pins.test_topk_ties_prefer_lower_index]),
    ("cdf_count", _cdf_strict, [pins.test_cdf_uniform_scores_closed_form]),
    ("attend_block", _attend_scale_squared, [pins.test_all_kept_equals_torch_sdpa_float64]),
    ("attend_block", _attend_values_from_keys, [pins.test_sparse_invariants]),
    ("attend_block", _attend_no_renormalise, [pins.test_sparse_invariants]),
    ("phi", _phi_plain_elu, [pins.test_phi_closed_form_and_elu]),
    ("phi", _phi_relu_plus_one, [pins.test_phi_closed_form_and_elu]),
    ("linear_block", _linear_unnormalised, [pins.test_linear_constant_v_gives_constant]),
    ("linear_block", _linear_state_transposed, [pins.test_linear_equals_token_quadratic_form]),
    ("classify_row", _sla3_marginal_from_bottom, [pins.test_sla3_invariants]),
]


@pytest.mark.parametrize("name,mutant,catchers", MUTANTS,
                         ids=[f"{n}:{m.__name__}" for n, m, _ in MUTANTS])
def test_pins_reject_mutant(monkeypatch, name, mutant, catchers):
    monkeypatch.setattr(sla, name, mutant)
    for catch in catchers:
        args = []
        if catch is pins.test_two_by_two_block_grid_all_masks:
            args = [2]
        with pytest.raises(AssertionError):
            catch(*args)


def test_unmutated_oracle_passes_the_same_pins():
    for _, _, catchers in MUTANTS:
        for catch in catchers:
            catch()
    assert math.isfinite(1.0)
