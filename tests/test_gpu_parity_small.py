"""GPU parity on small workloads that span several tiles and a ragged last block.

Every stage of the path is compared with the fp64 oracle through the C ABI:
pooled Q/K (fp32 diagnostic), class map and lists (bit-exact), the sparse
branch and its LSE, the linear branch, and the combined output (bars on the
fp32 pre-rounding output; the bf16 output must be its exact RNE rounding).
Where a linear branch exists, the fused call (prepare + sparse_linear_attn)
is held to the same bars and to the unfused sum.
"""

from fractions import Fraction as F

import numpy as np
import pytest
import torch

import block_sparse_attention_meanpool_amd as sla
from gpu_util import (REL_L2, bits_of, check_close, check_lse, counts, f64, rne_bf16_bits, say, small_inputs, to_dev)
from oracle import sla as osla
from synth.configs import Spec

pytestmark = pytest.mark.gpu

SMALL = [
    Spec(101, "iid_topk_d64_b64", B=2, H=2, N=1000, d=64, block=64, kind="iid", mode="topk",
         keep=F(1, 4)),
    Spec(102, "sla3_d128_b128", B=1, H=3, N=1000, d=128, block=128, kind="fourier",
         grid=(10, 10, 10), mode="sla3", keep=F(2, 8), marg=F(3, 8)),
    Spec(103, "cdf_d64_b128", B=1, H=2, N=1280, d=64, block=128, kind="fourier", grid=(4, 16, 20),
         mode="cdf", thr=0.2),
    Spec(104, "sla3_d128_b64", B=1, H=2, N=1200, d=128, block=64, kind="fourier", grid=(5, 12, 20),
         mode="sla3", keep=F(3, 19), marg=F(4, 19)),
    Spec(105, "topk_d128_b128_exact", B=1, H=2, N=1024, d=128, block=128, kind="fourier",
         grid=(4, 16, 16), mode="topk", keep=F(3, 8)),
    Spec(106, "cdf_d128_b128", B=1, H=2, N=1500, d=128, block=128, kind="fourier", grid=(5, 15, 20),
         mode="cdf", thr=0.1),
    # two batches through the pipelined kernel, the linear branch and the fused path; the last
    # block holds 60 tokens, so its second 64-key half is empty
    Spec(107, "sla3_d128_b128_two_batches", B=2, H=2, N=700, d=128, block=128, kind="fourier",
         grid=(7, 10, 10), mode="sla3", keep=F(2, 6), marg=F(2, 6)),
    # an odd number of key tiles (the linear-branch states go in pairs) with a ragged last one
    Spec(108, "sla3_d128_b128_odd_tiles", B=1, H=2, N=1100, d=128, block=128, kind="fourier",
         grid=(11, 10, 10), mode="sla3", keep=F(2, 9), marg=F(3, 9)),
]


@pytest.fixture(scope="module", params=SMALL, ids=[s.name for s in SMALL])
def case(request):
    spec = request.param
    say(f"[small parity] {spec.name}: B={spec.B} H={spec.H} N={spec.N} d={spec.d} b={spec.block}")
    data = small_inputs(spec)
    q64, k64, v64 = (osla.bf16_to_f64(data[t]) for t in "qkv")
    sel = spec.mode
    kc, km = counts(spec)
    cls_ref, s_ref, qp_ref, kp_ref = osla.class_map(q64, k64, spec.block, sel, spec.keep, spec.marg,
                                                    spec.thr)
    ref = osla.forward(q64, k64, v64, cls_ref, spec.block)
    q, k, v = (to_dev(data[t]) for t in "qkv")
    B, H, N, d, b, nb = spec.B, spec.H, spec.N, spec.d, spec.block, spec.nb
    qp = torch.empty((B, H, nb, d), dtype=torch.float32, device="cuda")
    kp = torch.empty_like(qp)
    cls = sla.sla_pool_classify(q, k, b, sel, kc, km, spec.thr or 0.0, q_pool=qp, k_pool=kp)
    kc_max = nb if sel == "cdf" else kc
    crit_idx, crit_cnt, marg_idx, marg_cnt = sla.sla_block_mask(cls, kc_max, km)
    o_s, lse = sla.sla_sparse_attn_fwd(q, k, v, b, crit_idx, crit_cnt, o_fp32=True, want_lse=True)
    o_s16, _ = sla.sla_sparse_attn_fwd(q, k, v, b, crit_idx, crit_cnt, o_fp32=False)
    o_lin = sla.sla_linear_branch_fwd(q, k, v, b, marg_idx, marg_cnt) if km else None
    o = sla.sla_combine(o_s, o_lin)
    fused32 = fused16 = None
    if km:
        lin_ws = sla.sla_linear_branch_prepare(k, v, b, marg_idx, marg_cnt)
        fused32, _ = sla.sla_sparse_linear_attn_fwd(q, k, v, b, crit_idx, crit_cnt, lin_ws,
                                                    o_fp32=True)
        fused16, _ = sla.sla_sparse_linear_attn_fwd(q, k, v, b, crit_idx, crit_cnt, lin_ws)
        fused32, fused16 = fused32.cpu().numpy(), bits_of(fused16)
    torch.cuda.synchronize()
    return dict(spec=spec, kc=kc, km=km, kc_max=kc_max, cls_ref=cls_ref, qp_ref=qp_ref,
                kp_ref=kp_ref, fused32=fused32, fused16=fused16, ref=ref, qp=f64(qp), kp=f64(kp), cls=cls.cpu().numpy(),
                crit_idx=crit_idx.cpu().numpy(), crit_cnt=crit_cnt.cpu().numpy(),
                marg_idx=None if marg_idx is None else marg_idx.cpu().numpy(),
                marg_cnt=None if marg_cnt is None else marg_cnt.cpu().numpy(),
                o_s=o_s.cpu().numpy(), lse=lse.cpu().numpy(), o_s16=bits_of(o_s16),
                o_lin=None if o_lin is None else o_lin.cpu().numpy(), o=bits_of(o))


def test_pooled_qk(case):
    for got, want, what in ((case["qp"], case["qp_ref"], "q_pool"), (case["kp"], case["kp_ref"], "k_pool")):
        err = np.abs(got - want).max()
        say(f"  {what}: max|d| = {err:.2e}")
        assert err <= 1e-5 * max(1.0, np.abs(want).max())


def test_class_map_bit_exact(case):
    np.testing.assert_array_equal(case["cls"], case["cls_ref"])


def test_lists_bit_exact(case):
    idx, cnt = osla.index_lists(case["cls_ref"], osla.CRITICAL, case["kc_max"])
    np.testing.assert_array_equal(case["crit_idx"], idx)
    np.testing.assert_array_equal(case["crit_cnt"], cnt)
    if case["km"]:
        idx, cnt = osla.index_lists(case["cls_ref"], osla.MARGINAL, case["km"])
        np.testing.assert_array_equal(case["marg_idx"], idx)
        np.testing.assert_array_equal(case["marg_cnt"], cnt)


def test_sparse_branch(case):
    o_s_ref, lse_ref, _, _ = case["ref"]
    check_close(case["o_s"], o_s_ref, "O_s")
    check_lse(case["lse"], lse_ref)
    # the bf16-output mode of the same kernel is the RNE rounding of its fp32 output
    np.testing.assert_array_equal(case["o_s16"], rne_bf16_bits(case["o_s"]))


def test_linear_branch(case):
    if not case["km"]:
        pytest.skip("no marginal blocks in this workload")
    _, _, o_lin_ref, _ = case["ref"]
    check_close(case["o_lin"], o_lin_ref, "O_lin")


def test_combined_output(case):
    _, _, _, o_ref = case["ref"]
    pre = case["o_s"] if case["o_lin"] is None else (case["o_s"] + case["o_lin"]).astype(np.float32)
    check_close(pre, o_ref, "O (fp32, pre-rounding)")
    np.testing.assert_array_equal(case["o"], rne_bf16_bits(pre))
    check_close(osla.bf16_to_f64(case["o"]), o_ref, "O (bf16)", max_abs=4e-2, rel_l2=8e-3)


def test_fused_output(case):
    if not case["km"]:
        pytest.skip("no marginal blocks in this workload")
    _, _, _, o_ref = case["ref"]
    f32 = case["fused32"]
    check_close(f32, o_ref, "O fused (fp32)")
    np.testing.assert_array_equal(case["fused16"], rne_bf16_bits(f32))
    # the same two fp32 branch outputs, summed without the intermediate rounding
    # of each: a few fp32 ulps of their magnitudes apart
    o_s, o_lin = case["o_s"].astype(np.float64), case["o_lin"].astype(np.float64)
    bound = 4 * 2.0 ** -24 * (np.abs(o_s) + np.abs(o_lin)) + 1e-30
    assert np.all(np.abs(f32 - (o_s + o_lin)) <= bound)
