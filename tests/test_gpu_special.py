"""GPU special cases: all-kept equals dense, constant V, empty rows, mask-in
edge cases, the device error flag, list order, and the forward() pipeline."""

import math
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import block_sparse_attention_meanpool_amd as sla
from gpu_util import BF16_U, REL_L2, check_lse, bits_of, check_close, f64, rne_bf16_bits, say, to_dev
from oracle import sla as osla
from synth import generate
from synth.configs import Spec

pytestmark = pytest.mark.gpu

SPEC = Spec(201, "special", B=1, H=2, N=1000, d=128, block=128, kind="fourier", grid=(10, 10, 10),
            mode="topk", keep=F(1, 2))


@pytest.fixture(scope="module")
def data():
    d = generate(SPEC, repairs=None, threads=1)
    return {t: d[t] for t in "qkv"}


def _lists_from(cls_np, width):
    idx, cnt = osla.index_lists(cls_np, osla.CRITICAL, width)
    return torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()


@pytest.mark.parametrize("d,block,N", [(128, 128, 1000), (64, 64, 700), (128, 64, 300), (64, 128, 520)])
def test_all_kept_equals_dense(d, block, N):
    say(f"[all kept] d={d} block={block} N={N}")
    g = np.random.default_rng(7)
    bits = [(g.standard_normal((1, 2, N, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            for _ in range(3)]
    q, k, v = (to_dev(x) for x in bits)
    nb = -(-N // block)
    cls = np.full((1, 2, nb, nb), osla.CRITICAL, dtype=np.uint8)
    idx, cnt = _lists_from(cls, nb)
    o_s, lse = sla.sla_sparse_attn_fwd(q, k, v, block, idx, cnt, o_fp32=True, want_lse=True)
    o_d, lse_d = sla.sla_dense_attn_fwd(q, k, v, block, o_fp32=True, want_lse=True)
    torch.cuda.synchronize()
    # the same core visits the same tiles in the same order
    assert torch.equal(o_s, o_d) and torch.equal(lse, lse_d)
    q64, k64, v64 = (osla.bf16_to_f64(x) for x in bits)
    o_ref, lse_ref, _, _ = osla.forward(q64, k64, v64, cls, block)
    check_close(o_s.cpu().numpy(), o_ref, "O_s vs dense oracle")
    check_lse(lse.cpu().numpy(), lse_ref)


def test_constant_v_gives_constant_output(data):
    q, k = to_dev(data["q"]), to_dev(data["k"])
    c = np.float32(1.625)
    vbits = np.full_like(data["v"], (np.array([c]).view(np.uint32) >> 16).astype(np.uint16)[0])
    v = to_dev(vbits)
    cls = sla.sla_pool_classify(q, k, 128, "topk", 4)
    idx, cnt, _, _ = sla.sla_block_mask(cls, 4)
    o_s, _ = sla.sla_sparse_attn_fwd(q, k, v, 128, idx, cnt, o_fp32=True)
    torch.cuda.synchronize()
    err = (o_s - float(c)).abs().max().item()
    # numerator (MFMA accumulation of bf16(p) * c) and normaliser (sum of the
    # same bf16(p)) differ only by fp32 accumulation order: <= c * n * 2^-23
    n_keys = 4 * 128
    say(f"  constant V: max|O - c| = {err:.2e}")
    assert err <= float(c) * n_keys * 2.0 ** -23


def test_mask_in_edge_rows_and_error_flag(data):
    q, k, v = (to_dev(data[t]) for t in "qkv")
    nb = SPEC.nb
    g = np.random.default_rng(3)
    cls = g.integers(0, 3, size=(1, 2, nb, nb)).astype(np.uint8)
    cls[0, 0, 0] = 0                       # a row with nothing kept
    cls[0, 0, 1] = osla.CRITICAL           # a row with everything critical
    cls[0, 1, 2] = osla.MARGINAL           # everything marginal
    cls[0, 1, 3, :] = 0
    cls[0, 1, 3, nb - 1] = osla.CRITICAL   # only the ragged last tile
    cls_d = torch.from_numpy(cls).cuda()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ci, cc, mi, mc = sla.sla_block_mask(cls_d, nb, nb, err_flag=flag)
    o_s, lse = sla.sla_sparse_attn_fwd(q, k, v, 128, ci, cc, o_fp32=True, want_lse=True)
    o_lin = sla.sla_linear_branch_fwd(q, k, v, 128, mi, mc)
    torch.cuda.synchronize()
    assert flag.item() == 0
    q64, k64, v64 = (osla.bf16_to_f64(data[t]) for t in "qkv")
    o_s_ref, lse_ref, o_lin_ref, _ = osla.forward(q64, k64, v64, cls, 128)
    o_s_np, lse_np = o_s.cpu().numpy(), lse.cpu().numpy()
    assert not o_s_np[0, 0, :128].any() and np.all(np.isneginf(lse_np[0, 0, :128]))
    assert not o_lin.cpu().numpy()[0, 0, 128:256].any()
    check_close(o_s_np, o_s_ref, "O_s (mask-in)")
    check_lse(lse_np, lse_ref, "LSE (mask-in)")
    check_close(o_lin.cpu().numpy(), o_lin_ref, "O_lin (mask-in)")


def test_error_flag_bad_class_and_overflow():
    nb = 8
    cls = np.zeros((1, 1, 4, nb), dtype=np.uint8)
    cls[0, 0, 0, 3] = 7                    # not a class
    cls[0, 0, 1, :5] = osla.CRITICAL       # 5 critical, width 3
    cls[0, 0, 2, [1, 6]] = osla.CRITICAL
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ci, cc, _, _ = sla.sla_block_mask(torch.from_numpy(cls).cuda(), 3, err_flag=flag)
    torch.cuda.synchronize()
    assert flag.item() == sla.FLAG_BAD_CLASS | sla.FLAG_OVERFLOW
    assert cc.cpu().tolist() == [[[0, 3, 2, 0]]]
    assert ci.cpu().numpy()[0, 0].tolist() == [[-1, -1, -1], [0, 1, 2], [1, 6, -1], [-1, -1, -1]]


def test_list_order_does_not_matter(data):
    q, k, v = (to_dev(data[t]) for t in "qkv")
    cls = sla.sla_pool_classify(q, k, 128, "topk", 4)
    idx, cnt, _, _ = sla.sla_block_mask(cls, 4)
    rev = torch.flip(idx, dims=[-1]).contiguous()
    a, _ = sla.sla_sparse_attn_fwd(q, k, v, 128, idx, cnt, o_fp32=True)
    b, _ = sla.sla_sparse_attn_fwd(q, k, v, 128, rev, cnt, o_fp32=True)
    torch.cuda.synchronize()
    # P is rounded to bf16 relative to the running maximum, which depends on
    # the visiting order: each weight moves by at most 2^-8 relative (bf16's
    # unit roundoff) in either order, so the outputs differ by at most
    # 2 * 2^-8 * max|V|
    vmax = float(np.abs(osla.bf16_to_f64(data["v"])).max())
    diff = (a - b).abs().max().item()
    say(f"  order: max|a - b| = {diff:.2e} (bound {2 * BF16_U * vmax:.2e})")
    assert diff <= 2 * BF16_U * vmax
    q64, k64, v64 = (osla.bf16_to_f64(data[t]) for t in "qkv")
    o_ref, _, _, _ = osla.forward(q64, k64, v64, cls.cpu().numpy(), 128)
    check_close(b.cpu().numpy(), o_ref, "O_s, descending list")


def test_marginal_list_repeats_and_strays(data):
    """A repeated marginal entry counts once and entries outside [0, nb) are
    ignored, in the standalone and the fused linear branch alike."""
    q, k, v = (to_dev(data[t]) for t in "qkv")
    nb = SPEC.nb
    cls = sla.sla_pool_classify(q, k, 128, "sla3", 2, 3)
    ci, cc, mi, mc = sla.sla_block_mask(cls, 2, 3)
    wide = torch.full(mi.shape[:-1] + (7,), -1, dtype=torch.int32, device="cuda")
    wide[..., :3] = mi
    wide[..., 3] = mi[..., 1]          # a repeat
    wide[..., 4] = nb + 5              # past the last block
    wide[..., 5] = -3
    wide[..., 6] = mi[..., 0]          # another repeat
    wc = torch.full_like(mc, 7)
    a = sla.sla_linear_branch_fwd(q, k, v, 128, mi, mc)
    b = sla.sla_linear_branch_fwd(q, k, v, 128, wide, wc)
    ws_a = sla.sla_linear_branch_prepare(k, v, 128, mi, mc)
    fa, _ = sla.sla_sparse_linear_attn_fwd(q, k, v, 128, ci, cc, ws_a, o_fp32=True)
    ws_b = sla.sla_linear_branch_prepare(k, v, 128, wide, wc)
    fb, _ = sla.sla_sparse_linear_attn_fwd(q, k, v, 128, ci, cc, ws_b, o_fp32=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(fa, fb)


def test_forward_pipeline_matches_stages(data):
    q, k, v = (to_dev(data[t]) for t in "qkv")
    out = sla.forward(q, k, v, 128, "sla3", keep=F(2, 8), marg=F(3, 8))
    cls = sla.sla_pool_classify(q, k, 128, "sla3", 2, 3)
    ci, cc, mi, mc = sla.sla_block_mask(cls, 2, 3)
    o_s, _ = sla.sla_sparse_attn_fwd(q, k, v, 128, ci, cc, o_fp32=True)
    o_lin = sla.sla_linear_branch_fwd(q, k, v, 128, mi, mc)
    o = sla.sla_combine(o_s, o_lin)
    torch.cuda.synchronize()
    assert torch.equal(out["cls"], cls)
    assert torch.equal(bits_of_t(out["o"]), bits_of_t(o))
    fused = sla.forward(q, k, v, 128, "sla3", keep=F(2, 8), marg=F(3, 8), fused=True)
    ws = sla.sla_linear_branch_prepare(k, v, 128, mi, mc)
    of, _ = sla.sla_sparse_linear_attn_fwd(q, k, v, 128, ci, cc, ws)
    torch.cuda.synchronize()
    assert torch.equal(bits_of_t(fused["o"]), bits_of_t(of))
    out2 = sla.forward(q, k, v, 128, "topk", keep=F(1, 4))
    o2, _ = sla.sla_sparse_attn_fwd(q, k, v, 128, out2["crit_idx"], out2["crit_cnt"], o_fp32=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_of(out2["o"]), rne_bf16_bits(o2.cpu().numpy()))


def bits_of_t(t):
    return t.view(torch.int16)
