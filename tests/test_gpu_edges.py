"""Degenerate lengths and the largest supported block count, through the C ABI.

* N from 1 token to a few blocks, with ragged last blocks, in all four (d,
  block) shapes and all three selection rules: class maps bit-exact, outputs
  within the bars; the backward of both branches at the smallest lengths in
  all four shapes.
* nb = 4096 key blocks (N = 524,288 at 128-token blocks, the ABI's limit):
  inputs built so that every row's pooled scores are strictly ordered by key
  block with gaps far above fp32 error (a ramp spread over two features, whose
  block means take exactly representable values); masks bit-exact, sampled
  outputs within the bars; and the selection at block counts that run each
  slot count of the top-k search.
"""

import math
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import block_sparse_attention_meanpool_amd as sla
from gpu_util import MAX_ABS, REL_L2, check_close, counts, say, small_inputs, to_dev
from oracle import grad as ograd
from oracle import sla as osla
from synth.configs import Spec
from synth.generate import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

CASES = [(1, 128, 128, "topk"), (1, 64, 64, "sla3"), (63, 64, 64, "topk"), (64, 128, 64, "sla3"),
         (65, 128, 64, "topk"), (127, 128, 128, "sla3"), (129, 128, 128, "topk"),
         (200, 64, 128, "cdf"), (300, 128, 64, "cdf")]


@pytest.mark.parametrize("N,d,block,mode", CASES)
def test_small_lengths(N, d, block, mode):
    spec = Spec(700 + N + d + block, "edge", B=1, H=2, N=N, d=d, block=block, kind="iid",
                mode=mode, keep=F(1, 2) if mode != "cdf" else None,
                marg=F(1, 4) if mode == "sla3" else None, thr=0.2 if mode == "cdf" else None)
    say(f"[edge] N={N} d={d} block={block} {mode}")
    data = small_inputs(spec)
    q64, k64, v64 = (osla.bf16_to_f64(data[t]) for t in "qkv")
    cls_ref, _, _, _ = osla.class_map(q64, k64, block, mode, spec.keep, spec.marg, spec.thr)
    q, k, v = (to_dev(data[t]) for t in "qkv")
    out = sla.forward(q, k, v, block, mode, keep=spec.keep, marg=spec.marg, thr=spec.thr,
                      o_fp32=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["cls"].cpu().numpy(), cls_ref)
    _, _, _, o_ref = osla.forward(q64, k64, v64, cls_ref, block)
    pre = out["o_s"] if "o_lin" not in out else out["o_s"] + out["o_lin"]
    check_close(pre.double().cpu().numpy(), o_ref, f"O N={N}")


@pytest.mark.parametrize("N,d,block", [(1, 128, 128), (127, 128, 128), (129, 128, 128),
                                       (1, 64, 64), (63, 64, 64), (65, 64, 64), (65, 128, 64),
                                       (129, 64, 128)])
def test_backward_small_lengths(N, d, block):
    say(f"[edge] backward, both branches, N={N}, d={d}, block={block}")
    g = np.random.default_rng(N + d + block)
    bits = [f32_to_bf16_bits(g.standard_normal((1, 2, N, d)).astype(np.float32)) for _ in range(4)]
    q, k, v, d_o = (to_dev(x) for x in bits)
    nb = -(-N // block)
    cls = g.choice(np.array([0, 1, 2], dtype=np.uint8), size=(1, 2, nb, nb), p=[0.2, 0.4, 0.4])
    cls[0, 0, 0, 0] = osla.CRITICAL
    ci, cc = (torch.from_numpy(x).cuda() for x in osla.index_lists(cls, osla.CRITICAL, nb))
    mi, mc = (torch.from_numpy(x).cuda() for x in osla.index_lists(cls, osla.MARGINAL, nb))
    o_s, lse = sla.sla_sparse_attn_fwd(q, k, v, block, ci, cc, o_fp32=True, want_lse=True)
    dq, dk, dv = sla.sla_sparse_attn_bwd(q, k, v, block, ci, cc, o_s, lse, d_o)
    lin_ws = sla.sla_linear_branch_prepare(k, v, block, mi, mc)
    sla.sla_linear_branch_bwd(q, k, v, block, mi, mc, d_o, lin_ws, dq, dk, dv)
    torch.cuda.synchronize()
    f64 = [osla.bf16_to_f64(x) for x in bits]
    ref = ograd.backward(*f64[:3], cls, block, f64[3])
    for t, r, n in zip((dq, dk, dv), ref, ("dQ", "dK", "dV")):
        got = t.cpu().numpy()
        if np.abs(r).max() < 1e-9:
            # One key per query (N = 1): both branches return v whatever q and
            # k are, so the exact dQ and dK are 0; the kernels leave rounding
            # residue of D = dO . O against dO . v, bounded by the max-abs bar.
            say(f"  {n} N={N}: exact gradient 0, max|got| = {np.abs(got).max():.2e}")
            assert np.abs(got).max() <= MAX_ABS
            continue
        scale = max(1.0, float(np.abs(r).max()))
        check_close(got, r, f"{n} N={N}", max_abs=MAX_ABS * scale, rel_l2=REL_L2)


def _ramp_inputs(nb, block=128, d=128, seed=0):
    """Key block j: feature 0 is 64 on (j // 32) of its tokens, feature 1 is 0.5
    on (j % 32) * 4 of them, so on those features kbar_j = (j // 32) / 2 and
    (j % 32) / 64, which sum to j / 64: with query block i holding +-1 on both
    features (the sign alternates with i) and small noise elsewhere,
    scale * qbar . kbar moves by ~1.4e-3 per key block, monotone in j."""
    g = np.random.default_rng(seed)
    N = nb * block
    k = 0.05 * g.standard_normal((N, d)).astype(np.float32)
    q = 0.05 * g.standard_normal((N, d)).astype(np.float32)
    v = g.standard_normal((N, d)).astype(np.float32)
    for j in range(nb):
        rows = k[j * block:(j + 1) * block]
        rows[:, 0] = 0.0
        rows[:, 1] = 0.0
        rows[: j // 32, 0] = 64.0
        rows[: (j % 32) * 4, 1] = 0.5
        q[j * block:(j + 1) * block, :2] = 1.0 if j % 2 == 0 else -1.0
    return tuple(f32_to_bf16_bits(x)[None, None] for x in (q, k, v))


def test_largest_block_count():
    nb = 4096
    say(f"[edge] nb = {nb} key blocks, N = {nb * 128}")
    qb, kb, vb = _ramp_inputs(nb)
    q64, k64 = osla.bf16_to_f64(qb), osla.bf16_to_f64(kb)
    keep = F(1, 100)
    cls_ref, s_ref, _, _ = osla.class_map(q64, k64, 128, "topk", keep)
    kc = osla.count_from_fraction(keep, nb)
    q, k, v = (to_dev(x) for x in (qb, kb, vb))
    cls = sla.sla_pool_classify(q, k, 128, "topk", kc)
    ci, cc, _, _ = sla.sla_block_mask(cls, kc)
    o, lse = sla.sla_sparse_attn_fwd(q, k, v, 128, ci, cc, o_fp32=True, want_lse=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cls.cpu().numpy(), cls_ref)
    idx_ref, cnt_ref = osla.index_lists(cls_ref, osla.CRITICAL, kc)
    np.testing.assert_array_equal(ci.cpu().numpy(), idx_ref)
    rows = [(0, 0, i) for i in (0, 1, 2047, 2048, 4094, 4095)]
    v64 = osla.bf16_to_f64(vb)
    res = osla.forward_rows(q64, k64, v64, cls_ref, 128, rows)
    got = np.concatenate([o[0, 0, i * 128:(i + 1) * 128].cpu().numpy() for (_, _, i) in rows])
    want = np.concatenate([res[r][0] for r in rows])
    check_close(got, want, "O (sampled rows), nb = 4096")


@pytest.mark.parametrize("nb", [700, 1100, 1600, 2500])
def test_selection_slot_counts(nb):
    """The top-k search holds a row in 4 ... 64 key slots per lane, chosen by nb:
    these block counts run the 12, 24, 32 and 48 slot kernels.  Ramp inputs
    (strictly ordered scores, gaps far above fp32 error); top-k and the
    three-way split, class maps bit-exact."""
    say(f"[edge] selection with nb = {nb} key blocks")
    qb, kb, _ = _ramp_inputs(nb, seed=nb)
    q64, k64 = osla.bf16_to_f64(qb), osla.bf16_to_f64(kb)
    q, k = to_dev(qb), to_dev(kb)
    for mode, keep, marg in (("topk", F(1, 20), None), ("sla3", F(1, 20), F(1, 10))):
        cls_ref = osla.class_map(q64, k64, 128, mode, keep, marg)[0]
        kc, km = osla.selection_counts(mode, nb, keep, marg)
        cls = sla.sla_pool_classify(q, k, 128, mode, kc, km)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(cls.cpu().numpy(), cls_ref, err_msg=f"{mode}, nb = {nb}")
