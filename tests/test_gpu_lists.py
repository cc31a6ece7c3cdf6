"""Caller-supplied tile lists that are not in the canonical form (strictly
ascending, in range), through the C ABI.

Every call reads a list as the set of its in-range entries, each tile once, at
its first position.  So:
  * a sorted list with repeated and out-of-range entries mixed in gives the
    same bits as its canonical form (same tiles in the same order), in the
    softmax forward, both backward kernels and the linear branch;
  * a shuffled list gives the same set (a different summation order in the
    softmax branch): within the bars of the oracle evaluated on the class map
    of that set, and the same bits in the linear branch;
  * sla_check_lists flags each kind of violation with its bit,
    sla_check_row_order flags row orders that are not permutations, and the debug
    build (SLA_DEBUG_CHECKS) flags them on every call that reads lists.
"""

import ctypes
import os
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import block_sparse_attention_meanpool_amd as sla
from gpu_util import MAX_ABS, check_close, check_lse, say, to_dev
from oracle import grad as ograd
from oracle import sla as osla
from synth import generate
from synth.configs import Spec

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bf16_bits(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _lists(nb, H, seed, width):
    """Canonical lists of random tile sets, and two altered forms of them:
    sorted with repeats and out-of-range entries mixed in, and shuffled with
    the same extras.  Returns (canon, sorted_extra, shuffled_extra) as
    (idx, cnt) pairs of numpy arrays, and the class map of the sets."""
    g = np.random.default_rng(seed)
    cls = np.zeros((1, H, nb, nb), dtype=np.uint8)
    rows = {}
    for h in range(H):
        for i in range(nb):
            # up to nb - 4 tiles, so that with 4 extra entries a row still fits the
            # widest list the interface takes (nb entries); one row is empty
            n = int(g.integers(1, nb - 3)) if (h, i) != (0, 1) else 0
            s = np.sort(g.choice(nb, size=n, replace=False))
            cls[0, h, i, s] = osla.CRITICAL
            rows[h, i] = s
    out = []
    for kind in ("canon", "sorted", "shuffled"):
        idx = np.full((1, H, nb, width), -1, dtype=np.int32)
        cnt = np.zeros((1, H, nb), dtype=np.int32)
        for (h, i), s in rows.items():
            r = list(s)
            if kind != "canon" and len(r):
                extra = [int(g.choice(r)) for _ in range(2)]     # repeats
                r = sorted(r + extra)
                r.insert(int(g.integers(0, len(r) + 1)), nb + 3)  # out of range, both sides
                r.insert(int(g.integers(0, len(r) + 1)), -5)
                if kind == "shuffled":
                    g.shuffle(r)
            idx[0, h, i, :len(r)] = r
            cnt[0, h, i] = len(r)
        out.append((idx, cnt))
    return out, cls


@pytest.mark.parametrize("d,block", [(128, 128), (64, 64)])
def test_lists_are_sets(d, block):
    N = 1000 if block == 128 else 600
    spec = Spec(310, f"lists_d{d}_b{block}", B=1, H=2, N=N, d=d, block=block, kind="fourier",
                grid=(10, 10, N // 100), mode="topk", keep=F(1, 2))
    nb = spec.nb
    width = nb
    say(f"[lists] d={d} block={block} N={N}: repeats, out-of-range entries, shuffled order")
    data = generate(spec, repairs=None, threads=1)
    g = np.random.default_rng(7)
    do_bits = _bf16_bits(g.standard_normal((1, spec.H, N, d)).astype(np.float32))
    q, k, v, d_o = (to_dev(x) for x in (data["q"], data["k"], data["v"], do_bits))
    (canon, srt, shf), cls = _lists(nb, spec.H, 40 + d, width)

    def run(lst):
        idx, cnt = (torch.from_numpy(x).cuda() for x in lst)
        o, lse = sla.sla_sparse_attn_fwd(q, k, v, block, idx, cnt, o_fp32=True, want_lse=True)
        dq, dk, dv = sla.sla_sparse_attn_bwd(q, k, v, block, idx, cnt, o, lse, d_o)
        lin = sla.sla_linear_branch_fwd(q, k, v, block, idx, cnt)
        flag = sla.sla_check_lists(idx, cnt, nb)
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in (o, lse, dq, dk, dv, lin)], int(flag.item())

    ref, f0 = run(canon)
    got_s, f1 = run(srt)
    got_x, f2 = run(shf)
    assert f0 == 0
    both = sla.FLAG_LIST_RANGE | sla.FLAG_LIST_REPEAT
    assert f1 & both == both and f2 & both == both, (f1, f2)
    names = ("O_s", "LSE", "dQ", "dK", "dV", "O_lin")
    for a, b, n in zip(got_s, ref, names):
        np.testing.assert_array_equal(a, b, err_msg=f"{n}: sorted list with extras")
    say("  sorted with repeats and out-of-range entries: bit-identical to the canonical lists")
    # the linear branch (bit rows) does not depend on the order of a list; the
    # softmax gradients do through O_s and LSE (D = dO . O_s, P from LSE)
    np.testing.assert_array_equal(got_x[5], ref[5], err_msg="O_lin: shuffled list")
    q64, k64, v64, do64 = (osla.bf16_to_f64(x) for x in (data["q"], data["k"], data["v"], do_bits))
    o_ref, lse_ref, _, _ = osla.forward(q64, k64, v64, cls, block)
    check_close(got_x[0], o_ref, "O_s (shuffled list)")
    check_lse(got_x[1], lse_ref, "LSE (shuffled list)")
    gref = ograd.backward(q64, k64, v64, cls, block, do64, branches=("softmax",))
    for a, b, n in zip(got_x[2:5], gref, ("dQ", "dK", "dV")):
        check_close(a, b, f"{n} (shuffled list)", max_abs=MAX_ABS * max(1.0, float(np.abs(b).max())))
    # the linear branch on the same sets as marginal tiles
    cls_m = np.where(cls == osla.CRITICAL, osla.MARGINAL, osla.SKIP).astype(np.uint8)
    _, _, lin_ref, _ = osla.forward(q64, k64, v64, cls_m, block)
    check_close(got_x[5], lin_ref, "O_lin (shuffled list)")


def test_check_lists_flags():
    nb, width = 10, 6
    rows = [([1, 3, 5], 3, 0),
            ([1, 3, 3, 5], 4, sla.FLAG_LIST_REPEAT),
            ([2, 10, 11], 3, sla.FLAG_LIST_RANGE),
            ([-1, 4], 2, sla.FLAG_LIST_RANGE),
            ([4, 2, 7], 3, sla.FLAG_LIST_ORDER),
            ([4, 2, 4], 3, sla.FLAG_LIST_ORDER | sla.FLAG_LIST_REPEAT),
            ([1, 2, 3, 4, 5, 6], 7, sla.FLAG_LIST_COUNT),
            ([1, 2], -1, sla.FLAG_LIST_COUNT),
            ([0, 1, 2, 3, 4, 9], 6, 0),
            ([5, 5, 5, 5, 5, 5], 2, sla.FLAG_LIST_REPEAT)]
    say(f"[lists] sla_check_lists on {len(rows)} hand-built rows")
    for entries, count, want in rows:
        idx = np.full((1, width), -1, dtype=np.int32)
        idx[0, :len(entries)] = entries
        i_d = torch.from_numpy(idx).cuda()
        c_d = torch.tensor([count], dtype=torch.int32, device="cuda")
        got = int(sla.sla_check_lists(i_d, c_d, nb).item())
        assert got == want, (entries, count, got, want)
    # all rows in one call: the OR of their bits
    idx = np.full((len(rows), width), -1, dtype=np.int32)
    for r, (entries, _, _) in enumerate(rows):
        idx[r, :len(entries)] = entries
    cnt = torch.tensor([c for _, c, _ in rows], dtype=torch.int32, device="cuda")
    got = int(sla.sla_check_lists(torch.from_numpy(idx).cuda(), cnt, nb).item())
    want = 0
    for _, _, w in rows:
        want |= w
    assert got == want


def test_check_row_order_flags():
    """sla_check_row_order sets FLAG_ORDER_PERM exactly for the heads whose
    entries are not a permutation of their query blocks."""
    g = np.random.default_rng(5)
    cases = []
    for nqb in (1, 7, 591, 4096):
        perm = np.stack([g.permutation(nqb) for _ in range(4)]).astype(np.int32).reshape(2, 2, nqb)
        cases.append((f"permutations, nqb={nqb}", perm, 0))
        if nqb > 1:
            rep = perm.copy()
            rep[1, 0, nqb // 2] = rep[1, 0, 0]          # one repeat, one block missing
            cases.append((f"repeat, nqb={nqb}", rep, sla.FLAG_ORDER_PERM))
        for bad in (nqb, -1):
            oob = perm.copy()
            oob[0, 1, nqb - 1] = bad
            cases.append((f"entry {bad}, nqb={nqb}", oob, sla.FLAG_ORDER_PERM))
    say(f"[lists] sla_check_row_order on {len(cases)} orders")
    for what, order, want in cases:
        got = int(sla.sla_check_row_order(torch.from_numpy(order).cuda()).item())
        assert got == want, (what, got, want)
    # what sla_row_order writes always passes
    ci = torch.from_numpy(g.integers(0, 50, (2, 3, 50, 4)).astype(np.int32)).cuda()
    cc = torch.from_numpy(g.integers(0, 5, (2, 3, 50)).astype(np.int32)).cuda()
    assert int(sla.sla_check_row_order(sla.sla_row_order(ci, cc)).item()) == 0


def test_debug_build_flags_list_arguments():
    """The SLA_DEBUG_CHECKS build validates the lists of every call that reads
    them into its device flag; a canonical list leaves it at zero."""
    from block_sparse_attention_meanpool_amd.binding import _SIGS
    from block_sparse_attention_meanpool_amd.build import variant_lib
    path = variant_lib("debug")
    if not os.path.exists(path):
        pytest.skip("the debug-checks build is not built (build(variant='debug'))")
    say(f"[lists] debug-checks build {path}")
    lib = ctypes.CDLL(path)
    for name in ("sla_sparse_attn_fwd", "sla_linear_branch_fwd", "sla_debug_flag"):
        res, args = _SIGS[name]
        getattr(lib, name).restype = res
        getattr(lib, name).argtypes = args
    hip = ctypes.CDLL("libamdhip64.so.7")  # by soname: the HIP runtime already in this process
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    torch.cuda.synchronize()
    addr = lib.sla_debug_flag()
    assert addr, "the debug build returned no flag address"

    def flag(clear=False):
        torch.cuda.synchronize()
        x = ctypes.c_int32(0)
        if clear:
            assert hip.hipMemcpy(ctypes.c_void_p(addr), ctypes.byref(x), 4, 1) == 0  # H2D
            return 0
        assert hip.hipMemcpy(ctypes.byref(x), ctypes.c_void_p(addr), 4, 2) == 0     # D2H
        return x.value

    B, H, N, d, b = 1, 1, 512, 64, 64
    nb = 8
    g = torch.Generator().manual_seed(3)
    q, k, v = (torch.randn((B, H, N, d), generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(sla.lib().sla_linear_branch_ws_bytes(B, H, N, d, b), 1), dtype=torch.uint8,
                     device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call(entries):
        idx = torch.full((B, H, nb, 4), -1, dtype=torch.int32)
        cnt = torch.zeros((B, H, nb), dtype=torch.int32)
        for i in range(nb):
            idx[0, 0, i, :len(entries)] = torch.tensor(entries, dtype=torch.int32)
            cnt[0, 0, i] = len(entries)
        idx, cnt = idx.cuda(), cnt.cuda()
        flag(clear=True)
        assert lib.sla_sparse_attn_fwd(P(q), P(k), P(v), B, H, N, d, b, P(idx), P(cnt), 4, None, 0.125,
                                       P(o), 1, None, stream) == 0
        f_attn = flag()
        flag(clear=True)
        assert lib.sla_linear_branch_fwd(P(q), P(k), P(v), B, H, N, d, b, P(idx), P(cnt), 4, P(o),
                                         P(ws), ws.numel(), stream) == 0
        return f_attn, flag()

    assert call([0, 3, 5]) == (0, 0)
    assert call([0, 3, 3]) == (sla.FLAG_LIST_REPEAT,) * 2
    assert call([9, 1]) == (sla.FLAG_LIST_RANGE | sla.FLAG_LIST_ORDER,) * 2
    say("  canonical lists leave the flag at 0; repeats, range and order set their bits")

    # a row order given to the softmax call is checked as well (a repeated
    # entry: one block computed twice with the same result, one not at all)
    idx = torch.full((B, H, nb, 4), -1, dtype=torch.int32)
    idx[..., 0] = 0
    cnt = torch.ones((B, H, nb), dtype=torch.int32)
    idx, cnt = idx.cuda(), cnt.cuda()
    for order, want in ((list(range(nb))[::-1], 0), ([0, 1, 2, 3, 4, 5, 6, 0], sla.FLAG_ORDER_PERM)):
        ro = torch.tensor(order, dtype=torch.int32, device="cuda").view(B, H, nb)
        flag(clear=True)
        assert lib.sla_sparse_attn_fwd(P(q), P(k), P(v), B, H, N, d, b, P(idx), P(cnt), 4, P(ro),
                                       0.125, P(o), 1, None, stream) == 0
        assert flag() == want, (order, want)
    say("  a permutation as row order leaves the flag at 0; a repeat sets FLAG_ORDER_PERM")


@pytest.mark.parametrize("d,block,N", [(128, 128, 3000), (64, 64, 1500)])
def test_row_order_changes_only_the_schedule(d, block, N):
    """sla_row_order sorts each head's query blocks by the median entry of
    their lists (ties by index, empty rows last); run with that order, the
    forward (plain and fused with the linear branch) and the backward give the
    same bits as in the natural order."""
    spec = Spec(311, f"order_d{d}_b{block}", B=2, H=2, N=N, d=d, block=block, kind="fourier",
                grid=(10, 10, N // 100), mode="sla3", keep=F(1, 4), marg=F(1, 4))
    nb = spec.nb
    say(f"[lists] row order, d={d} block={block} N={N} (nb={nb})")
    data = generate(spec, repairs=None, threads=1)
    g = np.random.default_rng(17)
    do_bits = _bf16_bits(g.standard_normal((spec.B, spec.H, N, d)).astype(np.float32))
    q, k, v, d_o = (to_dev(x) for x in (data["q"], data["k"], data["v"], do_bits))
    kc, km = osla.selection_counts("sla3", nb, spec.keep, spec.marg)
    cls = sla.sla_pool_classify(q, k, block, "sla3", kc, km)
    cls[1, 1, 2] = osla.SKIP   # one row with no critical tile: it sorts last
    ci, cc, mi, mc = sla.sla_block_mask(cls, kc, km)
    order = sla.sla_row_order(ci, cc)
    torch.cuda.synchronize()
    # the order against its definition
    ci_np, cc_np, got = ci.cpu().numpy(), cc.cpu().numpy(), order.cpu().numpy()
    for bb in range(spec.B):
        for h in range(spec.H):
            key = [(int(ci_np[bb, h, i, cc_np[bb, h, i] // 2]) if cc_np[bb, h, i] > 0 else 4096, i)
                   for i in range(nb)]
            want = [i for _, i in sorted(key)]
            np.testing.assert_array_equal(got[bb, h], want)
    assert got[1, 1, -1] == 2
    assert not np.array_equal(got[0, 0], np.arange(nb))  # not the identity on these inputs

    lin_ws = sla.sla_linear_branch_prepare(k, v, block, mi, mc)
    outs = []
    for ro in (None, order):
        o_s, lse = sla.sla_sparse_attn_fwd(q, k, v, block, ci, cc, o_fp32=True, want_lse=True,
                                           row_order=ro)
        fused, _ = sla.sla_sparse_linear_attn_fwd(q, k, v, block, ci, cc, lin_ws, o_fp32=True,
                                                  row_order=ro)
        dq, dk, dv = sla.sla_sparse_attn_bwd(q, k, v, block, ci, cc, o_s, lse, d_o, row_order=ro)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (o_s, lse, fused, dq, dk, dv)])
    for a, b, n in zip(outs[0], outs[1], ("O_s", "LSE", "O fused", "dQ", "dK", "dV")):
        np.testing.assert_array_equal(a, b, err_msg=f"{n} with and without the row order")
    say("  the order sorts by median tile; every output identical with and without it")
