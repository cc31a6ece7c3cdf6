"""Plant plausible mistakes in the oracle's gradients (on the CPU) and check
that a pin of test_oracle_grad.py rejects each one."""

import numpy as np
import pytest

import test_oracle_grad as pins
from oracle import grad, sla

_orig = {n: getattr(grad, n) for n in ("attend_block_grad", "linear_block_grad", "dphi")}


def _softmax_grad(mutation):
    def f(q_rows, k, v, kept_blocks, b, scale, d_o):
        N = k.shape[0]
        toks = sla._tokens_of(kept_blocks, N, b)
        r, d = q_rows.shape
        if len(toks) == 0:
            return np.zeros((r, d)), toks, np.zeros((0, d)), np.zeros((0, v.shape[1]))
        o, _, p = sla.attend_block(q_rows, k, v, kept_blocks, b, scale, return_p=True)
        kt, vt = k[toks], v[toks]
        dv = p.T @ d_o
        dp = d_o @ vt.T
        delta = (d_o * o).sum(axis=1, keepdims=True)
        ds = p * dp if mutation == "no_delta" else p * (dp - delta)
        dq = scale * (ds @ (vt if mutation == "dq_from_v" else kt))
        dk = (1.0 if mutation == "dk_unscaled" else scale) * (ds.T @ q_rows)
        if mutation == "dv_from_dp":
            dv = p.T @ (d_o - delta)
        return dq, toks, dk, dv
    return f


def _linear_grad(mutation):
    def f(q_rows, k, v, marg_blocks, b, d_o):
        N = k.shape[0]
        toks = sla._tokens_of(marg_blocks, N, b)
        r, d = q_rows.shape
        if len(toks) == 0:
            return np.zeros((r, d)), toks, np.zeros((0, d)), np.zeros((0, v.shape[1]))
        km, vm = k[toks], v[toks]
        a, ph = sla.phi(q_rows), sla.phi(km)
        state, zeta = ph.T @ vm, ph.sum(axis=0)
        u, w = a @ state, a @ zeta
        o_lin = u / w[:, None]
        du = d_o / w[:, None]
        dw = -(d_o * o_lin).sum(axis=1) / w
        if mutation == "dw_sign":
            dw = -dw
        da = du @ (state if mutation == "state_untransposed" else state.T) + np.outer(dw, zeta)
        dq = da if mutation == "no_dphi_q" else da * grad.dphi(q_rows)
        dstate, dzeta = a.T @ du, a.T @ dw
        dph = vm @ dstate.T
        if mutation != "no_dzeta":
            dph = dph + dzeta[None, :]
        dv = ph @ dstate
        dk = dph * grad.dphi(km)
        return dq, toks, dk, dv
    return f


def _dphi_relu(x):
    return np.where(np.asarray(x) > 0, 1.0, 0.0)


MUTANTS = {
    "softmax_no_delta": ("attend_block_grad", _softmax_grad("no_delta")),
    "softmax_dq_from_v": ("attend_block_grad", _softmax_grad("dq_from_v")),
    "softmax_dk_unscaled": ("attend_block_grad", _softmax_grad("dk_unscaled")),
    "softmax_dv_from_dp": ("attend_block_grad", _softmax_grad("dv_from_dp")),
    "linear_dw_sign": ("linear_block_grad", _linear_grad("dw_sign")),
    "linear_state_untransposed": ("linear_block_grad", _linear_grad("state_untransposed")),
    "linear_no_dphi_q": ("linear_block_grad", _linear_grad("no_dphi_q")),
    "linear_no_dzeta": ("linear_block_grad", _linear_grad("no_dzeta")),
    "dphi_relu": ("dphi", _dphi_relu),
}


def _some_pin_fails():
    checks = (
        lambda: pins.elementwise_fd_error() < 1e-7,
        lambda: pins.directional_fd_error() < 1e-7,
        lambda: pins.dense_autograd_error() < 1e-12,
    )
    return any(not c() for c in checks)


def test_unmutated_passes():
    assert not _some_pin_fails()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(grad, attr, fn)
    assert _some_pin_fails(), name
