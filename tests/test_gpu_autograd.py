"""The autograd form of the path (sla_attention / SlaAttention) on the GPU.

Its forward must be the separate-call path of forward() bit for bit, and the
gradients it hands to autograd must be those of sla_sparse_attn_bwd plus
sla_linear_branch_bwd for the same output gradient, rounded to bf16 (the
inputs' dtype).  The gradients themselves are checked against the oracle in
test_gpu_backward.py.
"""

from fractions import Fraction as F

import numpy as np
import pytest
import torch

import block_sparse_attention_meanpool_amd as sla
from gpu_util import say, to_dev
from oracle import sla as osla
from synth import generate
from synth.configs import Spec

pytestmark = pytest.mark.gpu


def _leaf(bits):
    return to_dev(bits).requires_grad_(True)


def _case(spec, seed, **sel):
    data = generate(spec, repairs=None, threads=1)
    q, k, v = (_leaf(data[t]) for t in "qkv")
    o, lists = sla.sla_attention(q, k, v, spec.block, **sel)
    cls, ci, cc, mi, mc = lists
    ref = sla.forward(q.detach(), k.detach(), v.detach(), spec.block, cls=cls,
                      keep=sel.get("keep"), marg=sel.get("marg"), o_fp32=True)
    assert torch.equal(o.view(torch.int16), ref["o"].view(torch.int16)), "forward differs"

    g = torch.Generator().manual_seed(seed)
    w = torch.randn(o.shape, generator=g).to(torch.bfloat16).cuda()
    (o.float() * w.float()).sum().backward()

    # the same gradients from the entry points, for d_o = w
    qd, kd, vd = q.detach(), k.detach(), v.detach()
    o_s, lse = sla.sla_sparse_attn_fwd(qd, kd, vd, spec.block, ci, cc, o_fp32=True, want_lse=True)
    dq, dk, dv = sla.sla_sparse_attn_bwd(qd, kd, vd, spec.block, ci, cc, o_s, lse, w)
    if mi is not None:
        lin_ws = sla.sla_linear_branch_prepare(kd, vd, spec.block, mi, mc)
        sla.sla_linear_branch_bwd(qd, kd, vd, spec.block, mi, mc, w, lin_ws, dq, dk, dv)
    torch.cuda.synchronize()
    for t, want, n in ((q, dq, "dQ"), (k, dk, "dK"), (v, dv, "dV")):
        assert t.grad is not None and t.grad.dtype == torch.bfloat16, n
        assert torch.equal(t.grad.view(torch.int16), want.to(torch.bfloat16).view(torch.int16)), n
        say(f"  {n}: max |grad| = {t.grad.float().abs().max().item():.3e}, equal to the entry points")
    return lists


def test_autograd_sla3_selection():
    spec = Spec(311, "ag_sla3", B=1, H=2, N=1000, d=128, block=128, kind="fourier",
                grid=(10, 10, 10), mode="sla3", keep=F(1, 4), marg=F(1, 4))
    say("[autograd] SLA three-way selection, d=128, block=128, N=1000 (ragged)")
    lists = _case(spec, 1, mode="sla3", keep=spec.keep, marg=spec.marg)
    assert lists[3] is not None and int(lists[4].sum()) > 0


def test_autograd_given_mask_generic_shape():
    spec = Spec(312, "ag_mask", B=1, H=2, N=1000, d=64, block=64, kind="fourier",
                grid=(10, 10, 10), mode="topk", keep=F(1, 2))
    say("[autograd] given class map, d=64, block=64, N=1000 (generic kernels)")
    g = np.random.default_rng(3)
    nb = spec.nb
    cls = g.choice(np.array([osla.SKIP, osla.MARGINAL, osla.CRITICAL], dtype=np.uint8),
                   size=(1, spec.H, nb, nb), p=[0.4, 0.35, 0.25])
    cls[0, 0, 1] = osla.SKIP               # a row with nothing at all
    cls[0, 1, 3, :] = osla.MARGINAL        # a row with only marginal tiles
    _case(spec, 2, cls=torch.from_numpy(cls).cuda())


def test_autograd_topk_no_linear_branch():
    spec = Spec(313, "ag_topk", B=1, H=2, N=700, d=128, block=128, kind="fourier",
                grid=(7, 10, 10), mode="topk", keep=F(1, 2))
    say("[autograd] top-k selection (no marginal tiles), N=700")
    lists = _case(spec, 3, mode="topk", keep=spec.keep)
    assert lists[3] is None


def test_autograd_expanded_output_gradient():
    """o.sum() hands backward a broadcast (stride-0) gradient of ones."""
    spec = Spec(314, "ag_sum", B=1, H=2, N=600, d=128, block=128, kind="fourier",
                grid=(6, 10, 10), mode="sla3", keep=F(2, 5), marg=F(1, 5))
    say("[autograd] gradient of o.sum(), N=600")
    data = generate(spec, repairs=None, threads=1)
    q, k, v = (_leaf(data[t]) for t in "qkv")
    o, (cls, ci, cc, mi, mc) = sla.sla_attention(q, k, v, spec.block, mode="sla3", keep=spec.keep,
                                                 marg=spec.marg)
    o.sum().backward()
    qd, kd, vd = q.detach(), k.detach(), v.detach()
    ones = torch.ones(o.shape, dtype=torch.bfloat16, device=o.device)
    o_s, lse = sla.sla_sparse_attn_fwd(qd, kd, vd, spec.block, ci, cc, o_fp32=True, want_lse=True)
    dq, dk, dv = sla.sla_sparse_attn_bwd(qd, kd, vd, spec.block, ci, cc, o_s, lse, ones)
    lin_ws = sla.sla_linear_branch_prepare(kd, vd, spec.block, mi, mc)
    sla.sla_linear_branch_bwd(qd, kd, vd, spec.block, mi, mc, ones, lin_ws, dq, dk, dv)
    torch.cuda.synchronize()
    for t, want, n in ((q, dq, "dQ"), (k, dk, "dK"), (v, dv, "dV")):
        assert torch.equal(t.grad.view(torch.int16), want.to(torch.bfloat16).view(torch.int16)), n
