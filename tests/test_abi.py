"""The C ABI on the host: the library loads, exports every symbol include/sla.h
declares, and rejects bad arguments before enqueueing anything.

Argument validation runs on the host before any HIP call, so these tests need
no GPU; no call here reaches a kernel launch.
"""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sla.h")

pytestmark = pytest.mark.skipif(
    not os.path.exists(os.path.join(ROOT, "block_sparse_attention_meanpool_amd", "libsla.so")),
    reason="libsla.so not built (run __graft_entry__.build())")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:sla_status|size_t|const char\*|int32_t\*?)\s+(sla_\w+)\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def mod():
    import block_sparse_attention_meanpool_amd as m
    return m


def test_header_declares_the_five_path_calls():
    names = _declared()
    for n in ("sla_pool_classify", "sla_block_mask", "sla_sparse_attn_fwd", "sla_linear_branch_fwd",
              "sla_combine"):
        assert n in names


def test_every_declared_symbol_is_exported(mod):
    so = mod.LIB_PATH
    out = subprocess.run(["nm", "-D", "--defined-only", so], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (sla_\w+)$", out, flags=re.M))
    for n in _declared():
        assert n in exported, n
        assert n in mod.EXPORTS, n
    h = ctypes.CDLL(so)
    for n in _declared():
        assert getattr(h, n)


def test_status_strings_and_version(mod):
    assert mod.sla_status_string(0) == "ok"
    assert "aligned" in mod.sla_status_string(-3)
    assert mod.sla_status_string(-99) == "unknown status"
    assert mod.sla_version() >= 100


P = ctypes.c_void_p
GOOD = P(0x10000)        # aligned, never dereferenced: validation fails first
ODD = P(0x10008)


def _pc(lib, q=GOOD, k=GOOD, B=1, H=2, N=1024, d=64, block=64, mode=0, kc=4, km=0, thr=0.0,
        scale=0.125, qp=None, kp=None, cls=GOOD, ws=GOOD, ws_bytes=1 << 40):
    return lib.sla_pool_classify(q, k, B, H, N, d, block, mode, kc, km, thr, scale, qp, kp, cls, ws,
                                 ws_bytes, None)


def test_pool_classify_rejects_bad_arguments(mod):
    lib = mod.lib()
    assert _pc(lib, q=None) == -1
    assert _pc(lib, N=0) == -1
    assert _pc(lib, d=96) == -2
    assert _pc(lib, block=32) == -2
    assert _pc(lib, N=4096 * 64 + 1) == -2          # more than 4096 blocks
    assert _pc(lib, q=ODD) == -3
    assert _pc(lib, kc=0) == -1
    assert _pc(lib, kc=17) == -1                    # nb = 16
    assert _pc(lib, mode=2, kc=10, km=7) == -1      # k_crit + k_marg > nb
    assert _pc(lib, mode=1, thr=0.0) == -1
    assert _pc(lib, mode=1, thr=1.0) == -1
    assert _pc(lib, mode=7) == -1
    assert _pc(lib, scale=0.0) == -1
    assert _pc(lib, qp=GOOD) == -1                  # q_pool without k_pool
    assert _pc(lib, ws=None) == -4
    assert _pc(lib, ws_bytes=16) == -4


def test_workspace_sizes(mod):
    lib = mod.lib()
    # scores [2, 16, 16] fp32 = 2048 B, pooled 2 x [2, 16, 64] fp32 = 16384 B
    assert lib.sla_pool_classify_ws_bytes(1, 2, 1024, 64, 64, 1) == 2048
    assert lib.sla_pool_classify_ws_bytes(1, 2, 1024, 64, 64, 0) == 2048 + 16384
    assert lib.sla_pool_classify_ws_bytes(1, 2, 1024, 96, 64, 0) == 0
    # bf16 states H_j^T [8, 128*128], fp32 z_j [8, 128], bit rows [8, 2 words] (256-byte
    # aligned), fp32 zeta_i [8, 128], bf16 gathered S_i^T [8, 128*128]
    assert lib.sla_linear_branch_ws_bytes(1, 1, 1000, 128, 128) == \
        8 * 128 * 128 * 2 + 8 * 128 * 4 + 256 + 8 * 128 * 4 + 8 * 128 * 128 * 2
    # backward, every shape: D and LSE log2 e fp32 [2, 1024] each, column bits
    # [2, 16, 2 words], counts [2, 16], uint16 column lists [2, 16, 16] (each piece
    # 256-byte aligned)
    for d, b in ((64, 64), (128, 64)):
        assert lib.sla_sparse_attn_bwd_ws_bytes(1, 2, 1024, d, b) == 2 * 8192 + 256 + 256 + 1024
    # linear backward: dS_i and dH_j bf16 [2, 16, d*d], dzeta_i and dz_j fp32 [2, 16, d],
    # column bits [2, 16, 2 words], then the states' low parts and S_i as a hi + lo
    # pair, bf16 [2, 16, d*d] each
    assert lib.sla_linear_branch_bwd_ws_bytes(1, 2, 1024, 64, 64) == \
        2 * (2 * 16 * 64 * 64 * 2) + 2 * (2 * 16 * 64 * 4) + 256 + 3 * (2 * 16 * 64 * 64 * 2)
    assert lib.sla_linear_branch_bwd_ws_bytes(1, 2, 1024, 96, 64) == 0


def test_other_entry_points_reject_bad_arguments(mod):
    lib = mod.lib()
    # block mask
    assert lib.sla_block_mask(None, 1, 1, 4, 4, GOOD, GOOD, 2, None, None, 0, None, None) == -1
    assert lib.sla_block_mask(GOOD, 1, 1, 4, 4, GOOD, GOOD, 0, None, None, 0, None, None) == -1
    assert lib.sla_block_mask(GOOD, 1, 1, 4, 4, GOOD, GOOD, 5, None, None, 0, None, None) == -1
    assert lib.sla_block_mask(GOOD, 1, 1, 4, 4, GOOD, GOOD, 2, GOOD, None, 2, None, None) == -1
    assert lib.sla_block_mask(GOOD, 1, 1, 4, 4, GOOD, GOOD, 2, GOOD, GOOD, 0, None, None) == -1
    # sparse attention
    sa = lib.sla_sparse_attn_fwd
    assert sa(GOOD, GOOD, GOOD, 1, 1, 256, 64, 64, None, GOOD, 2, None, 0.125, GOOD, 1, None, None) == -1
    assert sa(GOOD, GOOD, GOOD, 1, 1, 256, 64, 64, GOOD, GOOD, 5, None, 0.125, GOOD, 1, None, None) == -1
    assert sa(GOOD, GOOD, ODD, 1, 1, 256, 64, 64, GOOD, GOOD, 2, None, 0.125, GOOD, 1, None, None) == -3
    assert sa(GOOD, GOOD, GOOD, 1, 1, 256, 80, 64, GOOD, GOOD, 2, None, 0.125, GOOD, 1, None, None) == -2
    # a row order must be 4-byte aligned
    assert sa(GOOD, GOOD, GOOD, 1, 1, 256, 64, 64, GOOD, GOOD, 2, P(0x10002), 0.125, GOOD, 1, None,
              None) == -3
    # the row order call
    ro = lib.sla_row_order
    assert ro(None, GOOD, 1, 1, 4, 2, GOOD, None) == -1
    assert ro(GOOD, GOOD, 1, 1, 4097, 2, GOOD, None) == -1
    assert ro(GOOD, GOOD, 1, 1, 4, 0, GOOD, None) == -1
    assert ro(GOOD, GOOD, 1, 1, 4, 2, P(0x10001), None) == -3
    # dense baseline
    assert lib.sla_dense_attn_fwd(GOOD, GOOD, GOOD, 1, 1, 0, 64, 64, 0.125, GOOD, 1, None, None) == -1
    # linear branch
    lb = lib.sla_linear_branch_fwd
    assert lb(GOOD, GOOD, GOOD, 1, 1, 256, 64, 64, GOOD, GOOD, 2, GOOD, None, 0, None) == -4
    assert lb(GOOD, GOOD, GOOD, 1, 1, 256, 64, 64, GOOD, GOOD, 0, GOOD, GOOD, 1 << 40, None) == -1
    assert lb(GOOD, GOOD, GOOD, 1, 1, 256, 64, 64, GOOD, GOOD, 2, ODD, GOOD, 1 << 40, None) == -3
    # linear prepare
    lp = lib.sla_linear_branch_prepare
    assert lp(GOOD, GOOD, 1, 1, 256, 64, 64, GOOD, GOOD, 2, None, 0, None) == -4
    assert lp(GOOD, GOOD, 1, 1, 256, 64, 64, GOOD, GOOD, 2, GOOD, 16, None) == -4
    assert lp(None, GOOD, 1, 1, 256, 64, 64, GOOD, GOOD, 2, GOOD, 1 << 40, None) == -1
    assert lp(GOOD, GOOD, 1, 1, 256, 64, 64, GOOD, GOOD, 5, GOOD, 1 << 40, None) == -1
    assert lp(GOOD, ODD, 1, 1, 256, 64, 64, GOOD, GOOD, 2, GOOD, 1 << 40, None) == -3
    assert lp(GOOD, GOOD, 1, 1, 256, 96, 64, GOOD, GOOD, 2, GOOD, 1 << 40, None) == -2
    # fused sparse + linear
    fz = lib.sla_sparse_linear_attn_fwd
    args = [GOOD, GOOD, GOOD, 1, 1, 256, 64, 64, GOOD, GOOD, 2, None, 0.125, GOOD, 1 << 40, GOOD, 0,
            None, None]
    # every call below fails validation before anything is launched
    for pos, val, want in ((13, None, -4), (14, 16, -4), (15, None, -1), (8, None, -1),
                           (10, 5, -1), (12, 0.0, -1), (15, ODD, -3), (6, 80, -2),
                           (11, P(0x10002), -3)):
        bad = list(args)
        bad[pos] = val
        assert fz(*bad) == want, (pos, val)
    # combine
    assert lib.sla_combine(GOOD, 1, None, GOOD, 12, None) == -1
    assert lib.sla_combine(GOOD, 1, ODD, GOOD, 16, None) == -3
    assert lib.sla_combine(None, 1, None, GOOD, 16, None) == -1


def test_tile_permute_rejects_bad_arguments(mod):
    lib = mod.lib()
    tp = lib.sla_tile_permute

    def tiles(*shapes):
        flat = [t for shape in shapes for t in shape]
        return ctypes.cast((ctypes.c_int32 * len(flat))(*flat), ctypes.c_void_p)

    ok = tiles((1, 8, 8), (2, 4, 8))
    # grid 4 x 8 x 16, two heads, block 64
    assert tp(GOOD, GOOD, 1, 2, 4, 8, 16, 128, 64, ok, 0, None) == -1        # in place
    assert tp(GOOD, P(0x20000), 1, 2, 4, 8, 16, 128, 64, tiles((3, 8, 8), (2, 4, 8)), 0,
              None) == -1                                                   # 3 does not divide 4
    assert tp(GOOD, P(0x20000), 1, 2, 4, 8, 16, 128, 128, ok, 0, None) == -1  # volume != block
    assert tp(GOOD, P(0x20000), 1, 2, 4, 8, 16, 96, 64, ok, 0, None) == -2
    assert tp(ODD, P(0x20000), 1, 2, 4, 8, 16, 128, 64, ok, 0, None) == -3
    assert tp(GOOD, P(0x20000), 1, 2, 4, 8, 16, 128, 64, None, 0, None) == -1


def test_binding_refuses_cpu_tensors(mod):
    torch = pytest.importorskip("torch")
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mod.sla_pool_classify(q, q, 64, "topk", 1)


def test_counts_match_the_fraction_reading(mod):
    from fractions import Fraction as F
    assert mod.counts_for("topk", 591, F(5, 100)) == (30, 0)
    assert mod.counts_for("sla3", 256, F(5, 100), F(15, 100)) == (13, 39)
    assert mod.counts_for("sla3", 1920, F(10, 100), F(5, 100)) == (192, 96)
    assert mod.counts_for("cdf", 128) == (0, 0)


def test_list_validation_and_debug_flag_reject_bad_arguments(mod):
    lib = mod.lib()
    cl = lib.sla_check_lists
    assert cl(None, GOOD, 4, 2, 8, GOOD, None) == -1
    assert cl(GOOD, GOOD, 4, 2, 8, None, None) == -1
    assert cl(GOOD, GOOD, 0, 2, 8, GOOD, None) == -1
    assert cl(GOOD, GOOD, 4, 2, 4097, GOOD, None) == -1
    assert cl(GOOD, P(0x10002), 4, 2, 8, GOOD, None) == -3
    cp = lib.sla_clock_probe
    assert cp(None, 10, GOOD, None) == -1
    assert cp(GOOD, 10, None, None) == -1
    assert cp(GOOD, 0, GOOD, None) == -1
    assert cp(GOOD, 1000001, GOOD, None) == -1
    assert cp(P(0x10004), 10, GOOD, None) == -3
    co = lib.sla_check_row_order
    assert co(None, 1, 1, 8, GOOD, None) == -1
    assert co(GOOD, 1, 1, 8, None, None) == -1
    assert co(GOOD, 0, 1, 8, GOOD, None) == -1
    assert co(GOOD, 1, 1, 0, GOOD, None) == -1
    assert co(GOOD, 1, 1, 4097, GOOD, None) == -1
    assert co(P(0x10002), 1, 1, 8, GOOD, None) == -3
    assert co(GOOD, 1, 1, 8, P(0x10001), None) == -3
    # the release build keeps no debug flag
    if os.path.abspath(mod.LIB_PATH) == os.path.join(ROOT, "block_sparse_attention_meanpool_amd",
                                                     "libsla.so"):
        assert mod.debug_flag_address() is None


def test_noalloc_entry_point_rejects_bad_arguments(mod):
    lib = mod.lib()
    assert lib.sla_pool_classify_noalloc_scratch_bytes() == 80 << 20

    def call(q=GOOD, d=64, kc=4, mode=0, scale=0.125):
        return lib.sla_pool_classify_noalloc(q, GOOD, 1, 2, 1024, d, 64, mode, kc, 0, 0.0, scale,
                                             None, None, GOOD, None)
    assert call(q=None) == -1
    assert call(d=96) == -2
    assert call(q=ODD) == -3
    assert call(kc=0) == -1
    assert call(mode=9) == -1
    assert call(scale=0.0) == -1


def test_wrappers_reject_mismatched_shapes_before_any_device_use(mod):
    """Every buffer the library touches is sized from q's shape: the wrappers
    compare each given tensor's shape with it before anything else (these are
    CPU tensors, so a call that passed the shape checks would stop at the
    device check instead)."""
    import torch
    B, H, N, d, b = 1, 2, 300, 64, 64
    nb = 5
    bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32)
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)
    q, k, v = bf(B, H, N, d), bf(B, H, N, d), bf(B, H, N, d)
    ci, cc = i32(B, H, nb, 2), i32(B, H, nb)
    cases = [
        lambda: mod.sla_pool_classify(q, bf(B, H, N + 1, d), b, "topk", 1),
        lambda: mod.sla_pool_classify(q, k, b, "topk", 1, cls=torch.zeros((B, H, nb, nb + 1),
                                                                          dtype=torch.uint8)),
        lambda: mod.sla_pool_classify(q, k, b, "topk", 1, q_pool=f32(B, H, nb, d - 1),
                                      k_pool=f32(B, H, nb, d)),
        lambda: mod.sla_pool_classify_noalloc(q, k, b, "topk", 1, cls=torch.zeros((B, H, nb, 4),
                                                                                  dtype=torch.uint8)),
        lambda: mod.sla_block_mask(torch.zeros((B, H, nb, nb), dtype=torch.uint8), 2,
                                   crit_idx=i32(B, H, nb, 3), crit_cnt=cc),
        lambda: mod.sla_block_mask(torch.zeros((B, H, nb, nb), dtype=torch.uint8), 2, 2,
                                   crit_idx=ci, crit_cnt=cc, marg_idx=i32(B, H, nb, 2),
                                   marg_cnt=i32(B, H, nb - 1)),
        lambda: mod.sla_sparse_attn_fwd(q, k, bf(B, H, N, d + 1), b, ci, cc),
        lambda: mod.sla_sparse_attn_fwd(q, k, v, b, i32(B, H, nb + 1, 2), cc),
        lambda: mod.sla_sparse_attn_fwd(q, k, v, b, ci, i32(B, H, nb + 1)),
        lambda: mod.sla_sparse_attn_fwd(q, k, v, b, ci, cc, o_s=f32(B, H, N - 1, d)),
        lambda: mod.sla_sparse_attn_fwd(q, k, v, b, ci, cc, lse=f32(B, H, N + 1)),
        lambda: mod.sla_dense_attn_fwd(q, k, v, b, o=bf(B, H + 1, N, d)),
        lambda: mod.sla_linear_branch_fwd(q, k, v, b, ci, cc, o_lin=f32(B, H, N, 2 * d)),
        lambda: mod.sla_linear_branch_prepare(k, bf(B, H, N, 2 * d), b, ci, cc),
        lambda: mod.sla_sparse_linear_attn_fwd(q, k, v, b, ci, i32(B, H), torch.zeros(16, dtype=torch.uint8)),
        lambda: mod.sla_sparse_attn_bwd(q, k, v, b, ci, cc, f32(B, H, N, d), f32(B, H, N),
                                        bf(B, H, N - 2, d)),
        lambda: mod.sla_sparse_attn_bwd(q, k, v, b, ci, cc, f32(B, H, N, d), f32(B, H, N),
                                        bf(B, H, N, d), dk=f32(B, H, N, d + 2)),
        lambda: mod.sla_linear_branch_bwd(q, k, v, b, ci, cc, bf(B, H, N, d),
                                          torch.zeros(16, dtype=torch.uint8), f32(B, H, N, d),
                                          f32(B, H, N, d), f32(B, H, N + 1, d)),
        lambda: mod.sla_mask_recall(q, k, b, ci, cc, recall=f32(B, H, N, 1)),
        lambda: mod.sla_tile_permute(q, (3, 10, 10), [(1, 8, 8)] * H, b, y=bf(B, H, N, d + 8)),
        lambda: mod.sla_combine(f32(B, H, N, d), f32(B, H, N, d + 8)),
        lambda: mod.sla_check_lists(ci, i32(B, H, nb + 1), nb),
        lambda: mod.sla_check_row_order(i32(B, H)),
    ]
    for i, case in enumerate(cases):
        with pytest.raises(ValueError, match="shape") as e:
            case()
        assert "shape" in str(e.value), i
    # with consistent shapes the same CPU tensors stop at the device check
    with pytest.raises(ValueError, match="GPU tensor"):
        mod.sla_sparse_attn_fwd(q, k, v, b, ci, cc)
