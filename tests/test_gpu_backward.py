"""GPU parity of the backward pass (class map held fixed) against the oracle's
fp64 gradients (oracle/grad.py), through the C ABI.

Bars.  A gradient entry is a sum of products in which one factor (P or dS)
is rounded to bf16 (unit roundoff 2^-8) and everything else is exact bf16
input or fp32 accumulation; the rounding errors are independent, so the sum's
error is a few times 2^-9 of the magnitude of its terms.  The output bars
(rel-L2 5e-3, max-abs 2e-2) are therefore kept for every gradient, with the
max-abs bar taken relative to the gradient's scale:
|got - ref| <= 2e-2 * max(1, max |ref|), since dK and dV sum over every query
that attends a key and grow with that count.  The linear branch's dQ is the
difference of two terms that nearly cancel; the kernels give every factor
that enters one term rounded and the other not (S_i, O_lin, g) as a hi + lo
bf16 pair, so it is held to the same bars.
"""

from fractions import Fraction as F

import numpy as np
import pytest
import torch

import block_sparse_attention_meanpool_amd as sla
from gpu_util import MAX_ABS, REL_L2, check_close, say, to_dev
from oracle import grad as ograd
from oracle import sla as osla
from synth import generate
from synth.configs import Spec

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _grad_close(got, want, what, rel_l2=REL_L2):
    scale = max(1.0, float(np.abs(want).max()))
    return check_close(got, want, what, max_abs=MAX_ABS * scale, rel_l2=rel_l2)


def _rel_for(o_fp32):
    """The rel-L2 bar for a softmax-branch backward given O_s in fp32 (what the
    forward can write and the autograd form saves) or in bf16.  A bf16 O_s is
    an input of lower precision: D_n = dO_n . O_s_n then carries its rounding
    (up to 2^-9 |dO_n| |O_n|), and D enters every dS of the row, so dQ and dK
    inherit an error of the size of the rounding of O itself.  That input mode
    alone doubles the rel-L2 bar; every kernel-side rounding is held to 5e-3."""
    return REL_L2 if o_fp32 else 2 * REL_L2


def _dq_close(got, want, terms, what):
    """dQ at the plain bars; also prints how far below the size of its two
    cancelling terms (oracle.grad.linear_dq_scale) the error lies."""
    err, size = float(np.linalg.norm(got - want)), float(np.linalg.norm(terms))
    say(f"  {what}: |err| / |terms| = {err / max(size, 1e-30):.3e}")
    _grad_close(got, want, what)


def _mask(nb, H, seed, dense_frac=0.35):
    g = np.random.default_rng(seed)
    cls = np.where(g.random((1, H, nb, nb)) < dense_frac, osla.CRITICAL, osla.SKIP).astype(np.uint8)
    cls[0, 0, 0] = osla.CRITICAL           # a row with every tile
    cls[0, 0, 1] = osla.SKIP               # a row with none
    cls[0, 1, 2, :] = osla.SKIP
    cls[0, 1, 2, nb - 1] = osla.CRITICAL   # only the ragged last tile
    cls[0, 1, :, 3] = osla.SKIP            # a key tile no query block uses
    return cls


def _run(spec, cls, o_fp32=True, seed=5):
    data = generate(spec, repairs=None, threads=1)
    g = np.random.default_rng(seed)
    do_bits = _bf16_bits(g.standard_normal((spec.B, spec.H, spec.N, spec.d)).astype(np.float32))
    q, k, v, d_o = (to_dev(x) for x in (data["q"], data["k"], data["v"], do_bits))
    width = spec.nb
    idx, cnt = osla.index_lists(cls, osla.CRITICAL, width)
    idx_d, cnt_d = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    o_s, lse = sla.sla_sparse_attn_fwd(q, k, v, spec.block, idx_d, cnt_d, o_fp32=o_fp32,
                                       want_lse=True)
    dq, dk, dv = sla.sla_sparse_attn_bwd(q, k, v, spec.block, idx_d, cnt_d, o_s, lse, d_o)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = (osla.bf16_to_f64(x) for x in (data["q"], data["k"], data["v"], do_bits))
    ref = ograd.backward(q64, k64, v64, cls, spec.block, do64, branches=("softmax",))
    return (dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()), ref


SPEC = Spec(301, "bwd_small", B=1, H=2, N=1000, d=128, block=128, kind="fourier",
            grid=(10, 10, 10), mode="topk", keep=F(1, 2))


@pytest.mark.parametrize("o_fp32", [True, False], ids=["o_s_fp32", "o_s_bf16"])
def test_softmax_backward_small(o_fp32):
    say(f"[backward] softmax branch, N=1000 (ragged), o_s fp32={o_fp32}")
    cls = _mask(SPEC.nb, SPEC.H, 11)
    got, ref = _run(SPEC, cls, o_fp32)
    for a, b, n in zip(got, ref, ("dQ", "dK", "dV")):
        _grad_close(a, b, n, rel_l2=_rel_for(o_fp32))
    # the key tile no query block uses and the row with no tile get exactly nothing
    assert not got[1][0, 1, 3 * 128:4 * 128].any() and not got[2][0, 1, 3 * 128:4 * 128].any()
    assert not got[0][0, 0, 128:256].any()


@pytest.mark.parametrize("d,block,N", [(64, 64, 1000), (64, 128, 1000), (128, 64, 1000),
                                       (64, 64, 64), (128, 64, 200)])
def test_softmax_backward_other_shapes(d, block, N):
    """The generic kernels (every shape but d = 128 with 128-token blocks)."""
    nb = -(-N // block)
    spec = Spec(304, f"bwd_d{d}_b{block}", B=1, H=2, N=N, d=d, block=block, kind="fourier",
                grid=(1, 1, N) if N < 100 else (10, 10, N // 100), mode="topk", keep=F(1, 2))
    say(f"[backward] softmax branch, d={d}, block={block}, N={N} (nb={nb})")
    if nb >= 5:
        cls = _mask(nb, spec.H, 12)
    else:
        g = np.random.default_rng(13)
        cls = np.where(g.random((1, spec.H, nb, nb)) < 0.6, osla.CRITICAL, osla.SKIP).astype(np.uint8)
        cls[0, 0, 0] = osla.CRITICAL
    for o_fp32 in (True, False):
        got, ref = _run(spec, cls, o_fp32)
        for a, b, n in zip(got, ref, ("dQ", "dK", "dV")):
            _grad_close(a, b, f"{n} o_s fp32={o_fp32}", rel_l2=_rel_for(o_fp32))
    if nb >= 5:
        # the key tile no query block uses and the row with no tile get exactly nothing
        assert not got[1][0, 1, 3 * block:4 * block].any() and not got[2][0, 1, 3 * block:4 * block].any()
        assert not got[0][0, 0, block:2 * block].any()


def test_softmax_backward_selected_mask():
    spec = Spec(302, "bwd_topk", B=1, H=3, N=4000, d=128, block=128, kind="fourier",
                grid=(10, 20, 20), mode="topk", keep=F(1, 4))
    say("[backward] softmax branch, N=4000, top-k map from the GPU classifier")
    data = generate(spec, repairs=None, threads=1)
    q, k = to_dev(data["q"]), to_dev(data["k"])
    kc = osla.count_from_fraction(spec.keep, spec.nb)
    cls = sla.sla_pool_classify(q, k, spec.block, "topk", kc).cpu().numpy()
    got, ref = _run(spec, cls)
    for a, b, n in zip(got, ref, ("dQ", "dK", "dV")):
        _grad_close(a, b, n)


def _mask3(nb, H, seed):
    g = np.random.default_rng(seed)
    cls = g.choice(np.array([osla.SKIP, osla.MARGINAL, osla.CRITICAL], dtype=np.uint8),
                   size=(1, H, nb, nb), p=[0.4, 0.35, 0.25])
    cls[0, 0, 0] = osla.MARGINAL           # every tile marginal
    cls[0, 0, 1] = osla.SKIP               # nothing at all
    cls[0, 1, 2, :] = osla.SKIP
    cls[0, 1, 2, nb - 1] = osla.MARGINAL   # only the ragged last tile, marginal
    cls[0, 1, 3, :] = osla.CRITICAL        # no marginal tile at all
    cls[0, 1, :, 4] = osla.SKIP            # a key tile no query block uses
    return cls


def _run_both(spec, cls, branches, seed=9):
    data = generate(spec, repairs=None, threads=1)
    g = np.random.default_rng(seed)
    do_bits = _bf16_bits(g.standard_normal((spec.B, spec.H, spec.N, spec.d)).astype(np.float32))
    q, k, v, d_o = (to_dev(x) for x in (data["q"], data["k"], data["v"], do_bits))
    nb, b = spec.nb, spec.block
    ci, cc = (torch.from_numpy(x).cuda() for x in osla.index_lists(cls, osla.CRITICAL, nb))
    mi, mc = (torch.from_numpy(x).cuda() for x in osla.index_lists(cls, osla.MARGINAL, nb))
    if "softmax" in branches:
        o_s, lse = sla.sla_sparse_attn_fwd(q, k, v, b, ci, cc, o_fp32=True, want_lse=True)
        dq, dk, dv = sla.sla_sparse_attn_bwd(q, k, v, b, ci, cc, o_s, lse, d_o)
    else:
        dq, dk, dv = (torch.zeros(q.shape, dtype=torch.float32, device="cuda") for _ in range(3))
    lin_ws = sla.sla_linear_branch_prepare(k, v, b, mi, mc)
    sla.sla_linear_branch_bwd(q, k, v, b, mi, mc, d_o, lin_ws, dq, dk, dv)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = (osla.bf16_to_f64(x) for x in (data["q"], data["k"], data["v"], do_bits))
    ref = ograd.backward(q64, k64, v64, cls, b, do64, branches=branches)
    terms = ograd.linear_dq_scale(q64, k64, v64, cls, b, do64)
    return (dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()), ref, terms


def test_linear_backward_small():
    say("[backward] linear branch alone, N=1000 (ragged)")
    cls = _mask3(SPEC.nb, SPEC.H, 21)
    got, ref, terms = _run_both(SPEC, cls, ("linear",))
    # dK and dV have no cancelling difference: the plain bars
    _dq_close(got[0], ref[0], terms, "dQ")
    for a, b, n in zip(got[1:], ref[1:], ("dK", "dV")):
        _grad_close(a, b, n)
    assert not got[1][0, 1, 4 * 128:5 * 128].any() and not got[2][0, 1, 4 * 128:5 * 128].any()
    assert not got[0][0, 0, 128:256].any() and not got[0][0, 1, 3 * 128:4 * 128].any()


@pytest.mark.parametrize("d,block", [(64, 64), (64, 128), (128, 64)])
def test_linear_backward_other_shapes(d, block):
    """The generic linear-branch kernels, alone and after the softmax branch."""
    N = 1000
    spec = Spec(305, f"lbwd_d{d}_b{block}", B=1, H=2, N=N, d=d, block=block, kind="fourier",
                grid=(10, 10, 10), mode="topk", keep=F(1, 2))
    say(f"[backward] linear branch, d={d}, block={block}, N={N}")
    cls = _mask3(spec.nb, spec.H, 23)
    got, ref, terms = _run_both(spec, cls, ("linear",))
    _dq_close(got[0], ref[0], terms, "dQ")
    for a, b, n in zip(got[1:], ref[1:], ("dK", "dV")):
        _grad_close(a, b, n)
    assert not got[1][0, 1, 4 * block:5 * block].any() and not got[2][0, 1, 4 * block:5 * block].any()
    assert not got[0][0, 0, block:2 * block].any() and not got[0][0, 1, 3 * block:4 * block].any()
    got, ref, terms = _run_both(spec, cls, ("softmax", "linear"))
    _dq_close(got[0], ref[0], terms, "dQ (both)")
    for a, b, n in zip(got[1:], ref[1:], ("dK", "dV")):
        _grad_close(a, b, f"{n} (both)")


@pytest.mark.parametrize("d,block", [(128, 128), (64, 64)])
def test_backward_two_batches(d, block):
    """B = 2: every kernel indexes batch and head as one flattened dimension."""
    N = 700
    spec = Spec(306, f"bwd_b2_d{d}_b{block}", B=2, H=2, N=N, d=d, block=block, kind="fourier",
                grid=(7, 10, 10), mode="topk", keep=F(1, 2))
    say(f"[backward] both branches, B=2, d={d}, block={block}, N={N}")
    g = np.random.default_rng(24)
    nb = spec.nb
    cls = g.choice(np.array([osla.SKIP, osla.MARGINAL, osla.CRITICAL], dtype=np.uint8),
                   size=(2, spec.H, nb, nb), p=[0.4, 0.35, 0.25])
    cls[1, 1, 0] = osla.CRITICAL  # a row of the second batch with every tile critical
    cls[1, 0, 1] = osla.SKIP      # and one with nothing
    got, ref, terms = _run_both(spec, cls, ("softmax", "linear"))
    _dq_close(got[0], ref[0], terms, "dQ")
    for a, b, n in zip(got[1:], ref[1:], ("dK", "dV")):
        _grad_close(a, b, n)
    assert not got[0][1, 0, block:2 * block].any()


def test_both_branches_backward():
    spec = Spec(303, "bwd_sla3", B=1, H=2, N=2900, d=128, block=128, kind="fourier",
                grid=(10, 10, 29), mode="topk", keep=F(1, 2))
    say("[backward] both branches, N=2900 (ragged), sparse then linear accumulating")
    cls = _mask3(spec.nb, spec.H, 22)
    got, ref, terms = _run_both(spec, cls, ("softmax", "linear"))
    _dq_close(got[0], ref[0], terms, "dQ")
    for a, b, n in zip(got[1:], ref[1:], ("dK", "dV")):
        _grad_close(a, b, n)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,heads", [("tiny", (0, 1)), ("short_video", (0, 11)),
                                        ("wan1p3b", (0, 3, 7, 11)), ("wan14b", (0, 13, 39))])
def test_backward_workload(name, heads):
    """Full-size workloads: the GPU computes every head; the oracle checks the
    listed heads in full (all of their dQ, dK, dV)."""
    from synth import CONFIGS
    spec = CONFIGS[name]
    say(f"[backward workload] {name}: H={spec.H} N={spec.N}, checking heads {heads}")
    data = generate(spec)
    g = np.random.default_rng(31)
    do_bits = _bf16_bits(g.standard_normal((spec.B, spec.H, spec.N, spec.d), dtype=np.float32))
    q, k, v, d_o = (to_dev(x) for x in (data["q"], data["k"], data["v"], do_bits))
    b, nb = spec.block, spec.nb
    sel = "sla3" if spec.mode == "maskin" else spec.mode
    kc, km = osla.selection_counts(sel, nb, spec.keep, spec.marg)
    cls = sla.sla_pool_classify(q, k, b, sel, kc, km, spec.thr or 0.0)
    ci, cc, mi, mc = sla.sla_block_mask(cls, nb if sel == "cdf" else kc, km)
    o_s, lse = sla.sla_sparse_attn_fwd(q, k, v, b, ci, cc, o_fp32=True, want_lse=True)
    dq, dk, dv = sla.sla_sparse_attn_bwd(q, k, v, b, ci, cc, o_s, lse, d_o)
    branches = ("softmax",)
    if km:
        lin_ws = sla.sla_linear_branch_prepare(k, v, b, mi, mc)
        sla.sla_linear_branch_bwd(q, k, v, b, mi, mc, d_o, lin_ws, dq, dk, dv)
        branches = ("softmax", "linear")
    torch.cuda.synchronize()
    cls_np = cls.cpu().numpy()
    for h in heads:
        one = lambda x: osla.bf16_to_f64(x[0, h])[None, None]
        ref = ograd.backward(one(data["q"]), one(data["k"]), one(data["v"]), cls_np[:, h:h + 1], b,
                             one(do_bits), branches=branches)
        for t, r, n in zip((dq, dk, dv), ref, ("dQ", "dK", "dV")):
            _grad_close(t[0, h].cpu().numpy(), r[0, 0], f"{n} head {h}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,heads,n_tiles", [("long_clip_95", (0, 23), 3),
                                                ("long_clip_90", (0,), 2)])
def test_backward_long_clip_sampled(name, heads, n_tiles):
    """The 245,760-token layer (1920 blocks per head), both branches, in the
    launch configuration the benchmark times (row order on): the GPU computes
    every head; the oracle checks dQ of the first, the last and three seeded
    query blocks and dK, dV of the last and seeded key tiles of the listed
    heads (oracle.grad's samplers, equal to its whole backward on small
    cases). A whole head of the oracle's backward would take minutes here."""
    from synth import CONFIGS
    spec = CONFIGS[name]
    b, nb = spec.block, spec.nb
    say(f"[backward long clip] {name}: H={spec.H} N={spec.N}, heads {heads}")
    data = generate(spec)
    g = np.random.default_rng(37)
    do_bits = _bf16_bits(g.standard_normal((spec.B, spec.H, spec.N, spec.d), dtype=np.float32))
    q, k, v, d_o = (to_dev(x) for x in (data["q"], data["k"], data["v"], do_bits))
    kc, km = osla.selection_counts("sla3", nb, spec.keep, spec.marg)
    cls = sla.sla_pool_classify(q, k, b, "sla3", kc, km)
    ci, cc, mi, mc = sla.sla_block_mask(cls, kc, km)
    order = sla.sla_row_order(ci, cc)
    o_s, lse = sla.sla_sparse_attn_fwd(q, k, v, b, ci, cc, o_fp32=True, want_lse=True,
                                       row_order=order)
    dq, dk, dv = sla.sla_sparse_attn_bwd(q, k, v, b, ci, cc, o_s, lse, d_o, row_order=order)
    lin_ws = sla.sla_linear_branch_prepare(k, v, b, mi, mc)
    sla.sla_linear_branch_bwd(q, k, v, b, mi, mc, d_o, lin_ws, dq, dk, dv)
    torch.cuda.synchronize()
    del o_s, lse, lin_ws
    cls_np = cls.cpu().numpy()
    got = {n: [] for n in ("dQ", "dK", "dV")}
    want = {n: [] for n in ("dQ", "dK", "dV")}
    for h in heads:
        blocks = sorted({0, nb - 1, *(int(x) for x in g.integers(1, nb - 1, 3))})
        tiles = sorted({nb - 1, *(int(x) for x in g.integers(1, nb - 1, n_tiles - 1))})
        one = lambda x: osla.bf16_to_f64(x[0, h])
        args = (one(data["q"]), one(data["k"]), one(data["v"]), cls_np[0, h], b, one(do_bits))
        rows = ograd.backward_query_blocks(*args, blocks)
        cols = ograd.backward_key_tiles(*args, tiles)
        gq, gk, gv = (t[0, h].cpu().numpy() for t in (dq, dk, dv))
        for i in blocks:
            lo, hi = osla.block_bounds(spec.N, b, i)
            got["dQ"].append(gq[lo:hi])
            want["dQ"].append(rows[i])
        for j in tiles:
            lo, hi = osla.block_bounds(spec.N, b, j)
            got["dK"].append(gk[lo:hi])
            want["dK"].append(cols[j][0])
            got["dV"].append(gv[lo:hi])
            want["dV"].append(cols[j][1])
        say(f"  head {h}: query blocks {blocks}, key tiles {tiles} "
            f"(listed by {[int((cls_np[0, h, :, j] > 0).sum()) for j in tiles]} query blocks)")
    for n in ("dQ", "dK", "dV"):
        _grad_close(np.concatenate(got[n]), np.concatenate(want[n]), f"{n} (sampled)")
