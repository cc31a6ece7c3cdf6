"""GPU parity on the five workloads at their full sizes, through the C ABI.

Block masks (class map and lists) are compared bit-exactly in full.  Outputs
are compared on every query block for the two small workloads and on a
seeded sample of query blocks (always including the first and the last,
possibly ragged, block of each head) for the large ones, using the same
launches the benchmark times.  For the long-clip layer the mask is given as
input (the oracle's per-head top-k plus the next 5% as marginal), and the
GPU classifier is checked against it as well.
"""

import math
import time

import numpy as np
import pytest
import torch

import block_sparse_attention_meanpool_amd as sla
from gpu_util import REL_L2, check_close, check_lse, counts, f64, rne_bf16_bits, say, to_dev
from oracle import sla as osla
from synth import CONFIGS, generate

pytestmark = pytest.mark.gpu

FULL_OUTPUTS = ("tiny", "short_video")
SAMPLES_PER_HEAD = {"wan1p3b": 4, "wan14b": 2, "long_clip_95": 1, "long_clip_90": 1}


def _oracle_masks(spec, data):
    """Oracle class map, head by head (serially: numpy's BLAS must not be
    entered from several threads at once)."""
    sel = "sla3" if spec.mode == "maskin" else spec.mode

    def one(bh):
        b, h = bh
        q = osla.bf16_to_f64(data["q"][b, h])[None, None]
        k = osla.bf16_to_f64(data["k"][b, h])[None, None]
        cls, *_ = osla.class_map(q, k, spec.block, sel, spec.keep, spec.marg, spec.thr)
        return cls[0, 0]

    parts = [one((b, h)) for b in range(spec.B) for h in range(spec.H)]
    return np.stack(parts).reshape(spec.B, spec.H, spec.nb, spec.nb)


def _sample_rows(spec, n_per_head):
    g = np.random.default_rng(1000 + spec.cfg_id)
    rows = []
    for b in range(spec.B):
        for h in range(spec.H):
            pick = {0, spec.nb - 1}
            while len(pick) < min(spec.nb, 2 + n_per_head):
                pick.add(int(g.integers(0, spec.nb)))
            rows += [(b, h, i) for i in sorted(pick)]
    return rows


_cache = {}


def _data(spec):
    if spec.cfg_id not in _cache:
        _cache.clear()
        t0 = time.time()
        _cache[spec.cfg_id] = generate(spec)
        say(f"  generated cfg {spec.cfg_id} in {time.time() - t0:.1f} s")
    return _cache[spec.cfg_id]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny", "short_video", "wan1p3b", "wan14b", "long_clip_95",
                                  "long_clip_90"])
def test_workload_parity(name):
    spec = CONFIGS[name]
    say(f"[workload parity] {name}: B={spec.B} H={spec.H} N={spec.N} d={spec.d} b={spec.block} "
        f"mode={spec.mode}")
    data = _data(spec)
    t0 = time.time()
    cls_ref = _oracle_masks(spec, data)
    say(f"  oracle masks in {time.time() - t0:.1f} s")
    kc, km = counts(spec)
    sel = "sla3" if spec.mode == "maskin" else spec.mode
    q, k, v = (to_dev(data[t]) for t in "qkv")
    b = spec.block
    cls = sla.sla_pool_classify(q, k, b, sel, kc, km, spec.thr or 0.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cls.cpu().numpy(), cls_ref)
    say("  class map bit-exact")
    if spec.mode == "maskin":
        cls = torch.from_numpy(cls_ref).cuda()   # the mask is an input here
    kc_max = spec.nb if sel == "cdf" else kc
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ci, cc, mi, mc = sla.sla_block_mask(cls, kc_max, km, err_flag=flag)
    o_s, lse = sla.sla_sparse_attn_fwd(q, k, v, b, ci, cc, o_fp32=True, want_lse=True)
    o_lin = sla.sla_linear_branch_fwd(q, k, v, b, mi, mc) if km else None
    o = sla.sla_combine(o_s, o_lin)
    fused = None
    if km:
        lin_ws = sla.sla_linear_branch_prepare(k, v, b, mi, mc)
        fused, _ = sla.sla_sparse_linear_attn_fwd(q, k, v, b, ci, cc, lin_ws, o_fp32=True)
        del lin_ws
    torch.cuda.synchronize()
    assert flag.item() == 0
    idx_ref, cnt_ref = osla.index_lists(cls_ref, osla.CRITICAL, kc_max)
    np.testing.assert_array_equal(ci.cpu().numpy(), idx_ref)
    np.testing.assert_array_equal(cc.cpu().numpy(), cnt_ref)
    if km:
        idx_ref, cnt_ref = osla.index_lists(cls_ref, osla.MARGINAL, km)
        np.testing.assert_array_equal(mi.cpu().numpy(), idx_ref)
        np.testing.assert_array_equal(mc.cpu().numpy(), cnt_ref)
    say("  lists bit-exact; kept fraction "
        f"{cc.double().mean().item() / spec.nb:.4f}")

    if name in FULL_OUTPUTS:
        rows = [(bb, h, i) for bb in range(spec.B) for h in range(spec.H) for i in range(spec.nb)]
    else:
        rows = _sample_rows(spec, SAMPLES_PER_HEAD[name])
    t0 = time.time()
    got_s, got_lse, got_lin, got_o, want_s, want_lse, want_lin, want_o = ([] for _ in range(8))
    got_f = []
    heads = {}
    for (bb, h, i) in rows:
        if (bb, h) not in heads:
            heads.clear()
            heads[(bb, h)] = tuple(osla.bf16_to_f64(data[t][bb, h])[None, None] for t in "qkv")
        q64, k64, v64 = heads[(bb, h)]
        res = osla.forward_rows(q64, k64, v64, cls_ref[bb, h][None, None], b, [(0, 0, i)])
        r_s, r_lse, r_lin, r_o = res[(0, 0, i)]
        lo, hi = osla.block_bounds(spec.N, b, i)
        want_s.append(r_s); want_lse.append(r_lse); want_lin.append(r_lin); want_o.append(r_o)
        got_s.append(o_s[bb, h, lo:hi].cpu().numpy())
        got_lse.append(lse[bb, h, lo:hi].cpu().numpy())
        got_lin.append(np.zeros_like(r_lin) if o_lin is None else o_lin[bb, h, lo:hi].cpu().numpy())
        got_o.append(o[bb, h, lo:hi].cpu().contiguous().view(torch.int16).numpy().view(np.uint16))
        if fused is not None:
            got_f.append(fused[bb, h, lo:hi].cpu().numpy())
    say(f"  oracle outputs for {len(rows)} query blocks in {time.time() - t0:.1f} s")
    cat = np.concatenate
    check_close(cat(got_s), cat(want_s), "O_s")
    check_lse(cat(got_lse), cat(want_lse))
    if km:
        check_close(cat(got_lin), cat(want_lin), "O_lin")
    pre = (cat(got_s) + cat(got_lin)).astype(np.float32)
    check_close(pre, cat(want_o), "O (fp32, pre-rounding)")
    np.testing.assert_array_equal(cat(got_o), rne_bf16_bits(pre))
    check_close(osla.bf16_to_f64(cat(got_o)), cat(want_o), "O (bf16)", max_abs=4e-2, rel_l2=8e-3)
    if fused is not None:
        check_close(cat(got_f), cat(want_o), "O fused (fp32)")
