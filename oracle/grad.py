"""Gradients of the oracle forward with the class map held fixed (fp64).

TEST INFRASTRUCTURE ONLY (see the package header).

The SLA post ("results") says the method is trainable and needs only a short
fine-tuning; these are the gradients that training would use.  The block
selection is a discrete choice made before the attention, so it is held fixed:
the gradient flows through the two branches that the class map routes each
query block to, and the sum O = O_s + O_lin passes dO to both unchanged (R10).

Softmax branch, per query block with its critical tokens T (R11):
    P = softmax(scale Q K_T^T),  O_s = P V_T
    dV_T = P^T dO,   dP = dO V_T^T,   dS = P * (dP - rowsum(dO * O_s))
    dQ = scale dS K_T,   dK_T = scale dS^T Q

Linear branch, per query block with its marginal tokens M (R9):
    a = phi(Q), Phi = phi(K_M), S = Phi^T V_M, zeta = Phi^T 1
    u = a S, w = a zeta, O_lin = u / w
    dU = dO / w,   dw = -rowsum(dO * O_lin) / w
    da = dU S^T + dw zeta^T,      dQ = da * phi'(Q)
    dS = a^T dU,   dzeta = a^T dw
    dPhi = V_M dS^T + 1 dzeta^T,  dV_M = Phi dS,   dK_M = dPhi * phi'(K_M)
with phi'(x) = 1 for x > 0 and exp(x) otherwise.

Keys and values receive the sum over every query block whose lists contain
their tile.  A query block with an empty branch gets nothing from it (R12).
"""

import math

import numpy as np

from . import sla


def dphi(x):
    """Derivative of elu(x) + 1 (alpha = 1): 1 for x > 0, exp(x) otherwise."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def attend_block_grad(q_rows, k, v, kept_blocks, b, scale, d_o):
    """Gradient of the masked softmax attention of one query block.

    Returns (dq [r, d], toks, dk_toks [|T|, d], dv_toks [|T|, d]).
    """
    N = k.shape[0]
    toks = sla._tokens_of(kept_blocks, N, b)
    r, d = q_rows.shape
    if len(toks) == 0:
        z = np.zeros((0, d))
        return np.zeros((r, d)), toks, z, np.zeros((0, v.shape[1]))
    o, _, p = sla.attend_block(q_rows, k, v, kept_blocks, b, scale, return_p=True)
    kt, vt = k[toks], v[toks]
    dv = p.T @ d_o
    dp = d_o @ vt.T
    delta = (d_o * o).sum(axis=1, keepdims=True)
    ds = p * (dp - delta)
    dq = scale * (ds @ kt)
    dk = scale * (ds.T @ q_rows)
    return dq, toks, dk, dv


def linear_block_grad(q_rows, k, v, marg_blocks, b, d_o):
    """Gradient of the linear attention of one query block.

    Returns (dq [r, d], toks, dk_toks [|M|, d], dv_toks [|M|, d]).
    """
    N = k.shape[0]
    toks = sla._tokens_of(marg_blocks, N, b)
    r, d = q_rows.shape
    if len(toks) == 0:
        return np.zeros((r, d)), toks, np.zeros((0, d)), np.zeros((0, v.shape[1]))
    km, vm = k[toks], v[toks]
    a = sla.phi(q_rows)
    ph = sla.phi(km)
    state = ph.T @ vm
    zeta = ph.sum(axis=0)
    u = a @ state
    w = a @ zeta
    o_lin = u / w[:, None]
    du = d_o / w[:, None]
    dw = -(d_o * o_lin).sum(axis=1) / w
    da = du @ state.T + np.outer(dw, zeta)
    dq = da * dphi(q_rows)
    dstate = a.T @ du
    dzeta = a.T @ dw
    dph = vm @ dstate.T + dzeta[None, :]
    dv = ph @ dstate
    dk = dph * dphi(km)
    return dq, toks, dk, dv


def linear_dq_scale(q, k, v, cls, b, d_o):
    """Size of the terms of the linear branch's dQ (float64 [B, H, N, d]):
    (|dU| |S|^T + |dw| |zeta|^T) * |phi'(Q)| per query block, with the symbols
    of the header.

    dQ is the difference of dU S^T and dw zeta^T, which nearly cancel: when
    every value row is the same vector, O_lin equals it and dQ is exactly 0.
    A computation that rounds S or dU to a finite precision therefore errs in
    proportion to the size of these terms, not of their difference; this is
    that size, the scale a tolerance on dQ is measured against.
    """
    B, H, N, d = q.shape
    out = np.zeros_like(q)
    for bi in range(B):
        for h in range(H):
            for i in range(sla.num_blocks(N, b)):
                lo, hi = sla.block_bounds(N, b, i)
                toks = sla._tokens_of(np.nonzero(cls[bi, h, i] == sla.MARGINAL)[0], N, b)
                if len(toks) == 0:
                    continue
                a = sla.phi(q[bi, h, lo:hi])
                ph = sla.phi(k[bi, h, toks])
                state = ph.T @ v[bi, h, toks]
                zeta = ph.sum(axis=0)
                w = a @ zeta
                o_lin = (a @ state) / w[:, None]
                du = d_o[bi, h, lo:hi] / w[:, None]
                dw = -(d_o[bi, h, lo:hi] * o_lin).sum(axis=1) / w
                mag = np.abs(du) @ np.abs(state).T + np.outer(np.abs(dw), np.abs(zeta))
                out[bi, h, lo:hi] = mag * dphi(q[bi, h, lo:hi])
    return out


def backward(q, k, v, cls, b, d_o, scale=None, branches=("softmax", "linear")):
    """dQ, dK, dV (float64 [B, H, N, d]) of sum(O * d_o) with O from sla.forward.

    `branches` restricts the gradient to one branch (the same sum with the
    other branch's output held constant).
    """
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nqb = sla.num_blocks(N, b)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for bi in range(B):
        for h in range(H):
            for i in range(nqb):
                lo, hi = sla.block_bounds(N, b, i)
                qr, g = q[bi, h, lo:hi], d_o[bi, h, lo:hi]
                if "softmax" in branches:
                    crit = np.nonzero(cls[bi, h, i] == sla.CRITICAL)[0]
                    a, toks, ck, cv = attend_block_grad(qr, k[bi, h], v[bi, h], crit, b, scale, g)
                    dq[bi, h, lo:hi] += a
                    np.add.at(dk[bi, h], toks, ck)
                    np.add.at(dv[bi, h], toks, cv)
                if "linear" in branches:
                    marg = np.nonzero(cls[bi, h, i] == sla.MARGINAL)[0]
                    a, toks, ck, cv = linear_block_grad(qr, k[bi, h], v[bi, h], marg, b, g)
                    dq[bi, h, lo:hi] += a
                    np.add.at(dk[bi, h], toks, ck)
                    np.add.at(dv[bi, h], toks, cv)
    return dq, dk, dv


def backward_query_blocks(q, k, v, cls, b, d_o, blocks, scale=None,
                          branches=("softmax", "linear")):
    """dQ of the given query blocks of one head, as backward() computes them:
    {i: float64 [rows of block i, d]}, with q, k, v, d_o [N, d] and cls
    [nqb, nkb] of that head.  A query block's dQ depends only on its own rows
    and lists, so each is computed on its own (for layers too long to run
    backward() on every block)."""
    N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = {}
    for i in blocks:
        lo, hi = sla.block_bounds(N, b, i)
        qr, g = q[lo:hi], d_o[lo:hi]
        acc = np.zeros((hi - lo, d))
        if "softmax" in branches:
            crit = np.nonzero(cls[i] == sla.CRITICAL)[0]
            acc += attend_block_grad(qr, k, v, crit, b, scale, g)[0]
        if "linear" in branches:
            marg = np.nonzero(cls[i] == sla.MARGINAL)[0]
            acc += linear_block_grad(qr, k, v, marg, b, g)[0]
        out[i] = acc
    return out


def backward_key_tiles(q, k, v, cls, b, d_o, tiles, scale=None,
                       branches=("softmax", "linear")):
    """dK and dV of the given key tiles of one head, as backward() accumulates
    them: {j: (dk, dv)}, each float64 [rows of tile j, d].  A tile's rows
    receive the contribution of every query block whose critical (softmax) or
    marginal (linear) list holds it, summed in query-block order; only those
    query blocks are visited."""
    N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    tiles = list(tiles)
    bounds = {j: sla.block_bounds(N, b, j) for j in tiles}
    out = {j: (np.zeros((hi - lo, d)), np.zeros((hi - lo, v.shape[1])))
           for j, (lo, hi) in bounds.items()}
    kinds = [(sla.CRITICAL, "softmax"), (sla.MARGINAL, "linear")]
    for i in range(cls.shape[0]):
        lo, hi = sla.block_bounds(N, b, i)
        for cl, branch in kinds:
            if branch not in branches or not any(cls[i, j] == cl for j in tiles):
                continue
            kept = np.nonzero(cls[i] == cl)[0]
            if branch == "softmax":
                _, toks, ck, cv = attend_block_grad(q[lo:hi], k, v, kept, b, scale, d_o[lo:hi])
            else:
                _, toks, ck, cv = linear_block_grad(q[lo:hi], k, v, kept, b, d_o[lo:hi])
            for j in tiles:
                if cls[i, j] != cl:
                    continue
                tlo, thi = bounds[j]
                sel = (toks >= tlo) & (toks < thi)
                out[j][0][toks[sel] - tlo] += ck[sel]
                out[j][1][toks[sel] - tlo] += cv[sel]
    return out

